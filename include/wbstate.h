/*
 * wbstate.h -- C ABI of the quantized recurrent-state write-back library (MI355X, gfx950).
 *
 * One library call advances, converts or re-allocates the stored low-bit states of a
 * gated delta-rule (GDN / KDA) linear-attention layer on the GPU. Pages cited:
 *   [WB]     "When Quantization Breaks Memory: Recurrent-State Write-Back in
 *            Low-Precision Temporal Inference" (summary page) and its Chinese-language
 *            summary page [WB-zh];
 *   [LBRS]   "Low-Bit Recurrent States in Hybrid Language Models";
 *   [LBRS-x] "Allocate low-bit recurrent state precision by channel decay" (explainer);
 *   [DAMP]   summary page of "DAMP: Decay-Aware Mixed-Precision recurrent-state
 *            quantization".
 *
 * Conventions for every call
 *   - Return 0 (WB_OK) or a negative status (below); state_status_str() names it.
 *   - Device pointers are plain HIP device addresses owned by the caller; the library
 *     never allocates or frees device memory. Host pointers are read during the call.
 *   - Every device buffer must be 16-byte aligned (WB_EALIGN otherwise).
 *   - Arguments are validated on the host before anything is enqueued; a rejected call
 *     enqueues nothing. Accepted calls are asynchronous on `stream` (a hipStream_t;
 *     NULL is the default stream); execution errors surface at the caller's
 *     synchronisation. No call synchronises the host except state_alloc's copy of a
 *     permutation.
 *   - A handle must be used by one stream at a time; regions of different heads are
 *     independent, so every kernel updates its region in place without races.
 *   - Shapes: dk = dv = 128 for every layout; FP32 and UNIFORM also take dk = dv = 16.
 *
 * Tensor layouts (row-major, float32 unless stated):
 *   q, k   [B][H][dk]     query and key of the current token
 *   v      [B][H][dv]     value
 *   beta   [B][H]         write strength
 *   s      [B][H][dk] (decay WB_DECAY_PER_ROW, KDA) or [B][H] (WB_DECAY_PER_HEAD, GDN):
 *                         decay rate, the row factor being e^{-s}
 *   o      [B][H][dv]     readout o_t = S_t^T q_t
 *   S      [B][H][dk][dv] a state in the original domain and logical row order
 *
 * Stored state (device buffer of state_bytes()): B*H regions in order b*H + h, each
 * padded to a multiple of 256 bytes, followed (MIXED only) by the per-head row
 * permutation, uint8 [H][dk]. Region formats (little-endian):
 *   FP32      float32 [dk][dv].
 *   UNIFORM   `bits`-bit two's-complement level kappa of element (i, j) at bit offset
 *             bits*(i*dv + j), LSB first; value kappa * 2^(1-bits) ([WB-zh] "Core method":
 *             Delta_4 = 0.125 on [-1, 1]; rails at -1 and 1 - Delta).
 *   HAD_INT8  rows Hadamard-rotated along dv (orthonormal Sylvester, natural order):
 *             uint8 codes [dk][dv]; then (f16 scale, f16 zero) [dk][dv/block];
 *             value = zero + code * scale ([DAMP] "Quantization & calibration details").
 *   MIXED     physical row p holds logical row perm[h][p]; physical rows < k_hi are
 *             float16 [k_hi][dv]; the others are HAD_INT8 rows: uint8 codes
 *             [dk-k_hi][dv], then (f16 scale, f16 zero) [dk-k_hi][dv/block]
 *             ([DAMP] "Risk scoring and selection", "Implementation"; 9.875 bits per
 *             value at k_hi = 16, block = 32: [LBRS] "Related work").
 *   BITALLOC  row i's codes at byte (dv/8)*sum_{i'<i} b_i', element j at bits
 *             [j*b_i, (j+1)*b_i) as kappa + n_i, n_i = 2^(b_i-1) - 1; code area
 *             dk*dv*bbar/8 bytes; then f16 Delta [dk]; then uint8 meta [dk] =
 *             (b_i - 1) | (k_i << 4), k_i the clipping-fit index, f = 1/4 + k_i/20
 *             ([LBRS] "State bit allocation", "Levels and storage").
 * Error-feedback side buffer (mode WB_EF, every layout but FP32): float32
 * [B][H][dk][dv], physical row order, in the quantizer's (rotated) domain; entries of
 * MIXED float16 rows are neither read nor written.
 */
#ifndef WBSTATE_H
#define WBSTATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define WB_OK 0
#define WB_EINVAL (-1)        /* invalid argument (null pointer, bad enum, bad count) */
#define WB_ESIZE (-2)         /* a buffer is smaller than the layout needs */
#define WB_EUNSUPPORTED (-3)  /* shape / layout / mode combination not built */
#define WB_ELAUNCH (-4)       /* the HIP runtime refused a launch or copy */
#define WB_EALIGN (-5)        /* a device pointer is not 16-byte aligned */
#define WB_ESCRATCH (-6)      /* the work exceeds the library's static scratch (see
                               * state_allocate_bits_static) */

/* storage layouts */
#define WB_FP32 0      /* identity write-back, q_t = h_t */
#define WB_UNIFORM 1   /* uniform B-bit grid */
#define WB_HAD_INT8 2  /* Hadamard rows, per-block asymmetric affine INT8 */
#define WB_MIXED 3     /* k_hi float16 rows + Hadamard INT8 rows, static permutation */
#define WB_BITALLOC 4  /* decay-aware per-row widths, packed mixed-width codes */
#define WB_HEADALLOC 5 /* decay-aware per-head width, a float16 scale per 32 key channels of a
                        * column ([LBRS] "Allocation units"): element (i, j) at bits
                        * [(i dv + j) b, +b) as kappa + n, n = 2^(b-1) - 1, in a code area of
                        * dk*dv*bmax/8 bytes; then f16 Delta [dk/32][dv]; then u8 clipping-fit
                        * index [dk/32][dv]; then u8 (b - 1) and 15 zero bytes. Widths are
                        * budgeted over the heads of a sequence (budget must be 0). */

/* write-back rules ([WB] "Post-training write-back interventions and diagnostics";
 * [WB-zh] "Error feedback and stochastic rounding"). FP32 ignores the rule.
 * MIXED float16 rows always round to nearest. */
#define WB_RTN 0       /* nearest level, half-step ties to the even index, rail clamp */
#define WB_SR 1        /* stochastic rounding: floor(tau) + [r < frac(tau) * 2^16], r a 16-bit
                          Philox4x32-10 slice, key (seed lo, seed hi), counter
                          (16*row + col/8, b*H + h, t lo, t hi), column col using word
                          (col%8)/2, low half for even col */
#define WB_EF 2        /* error feedback: round (h + e), then e = clip(h + e - q, -step, step) */
#define WB_DIR 3       /* direction memory (UNIFORM only), k = mem_bits: a signed counter c per
                          element; with q the level entering the step and d = h - q: a change of
                          the nearest level is written as usual and resets c; otherwise
                          step/8 < |d| < step/2 adds sign(d) to c and, when |c| reaches 2^(k-1),
                          the level moves one step that way (clipped at the rails) and c resets
                          ([WB] "Interventions", "Post-training write-back interventions and
                          diagnostics", "Trajectory analysis") */
#define WB_RESQ 4      /* quantized residual memory (UNIFORM only), k = mem_bits: error feedback
                          whose carried residual clip(h + e - q, -step, step) is itself rounded
                          to the nearest j * step / 2^(k-1), j in [-2^(k-1), 2^(k-1) - 1], ties
                          to even j ([WB] "Post-training write-back interventions and
                          diagnostics": residual widths k = 2, 3, 4) */

#define WB_DECAY_PER_HEAD 0
#define WB_DECAY_PER_ROW 1

/* persistence factor Gamma_i of the bit allocation ([LBRS] "Approximate erasure rate",
 * "Choice of persistence factor", "Related work") */
#define WB_GAMMA_ERASURE 0  /* 1 / (C expm1(2 (s_i + r_i))), the approximate erasure rate */
#define WB_GAMMA_W1 1       /* 1 / (1 - a_i^2), a_i = e^{-s_i}: DAMP's factor, uncapped */
#define WB_GAMMA_HC 2       /* 1 / (1 - e^{-2 C s_i}): the write-back-time factor */

/* BITALLOC width budget ([LBRS] "State bit allocation": a layer-wise mean budget) */
#define WB_BUDGET_HEAD 0    /* each head's widths sum to bbar * dk; code area exactly full */
#define WB_BUDGET_LAYER 1   /* the widths of all H heads of a sequence sum to bbar * H * dk;
                             * each head's code area holds bmax * dk * dv / 8 bytes, zero
                             * after the head's last row */

typedef struct wb_layout_desc {
    int32_t kind;    /* WB_FP32 .. WB_BITALLOC */
    int32_t mode;    /* WB_RTN, WB_SR, WB_EF, WB_DIR, WB_RESQ */
    int32_t decay;   /* WB_DECAY_PER_HEAD or WB_DECAY_PER_ROW */
    int32_t B, H, dk, dv;
    int32_t bits;    /* UNIFORM level width: 2, 4 or 8 */
    int32_t block;   /* HAD_INT8 / MIXED affine block length along dv: 32, 64 or 128 */
    int32_t k_hi;    /* MIXED float16 rows: a positive multiple of dk/8 below dk */
    int32_t bbar, bmin, bmax;  /* BITALLOC mean width and clip range, 2 <= bmin <= bbar <= bmax <= 8 */
    int32_t mem_bits;          /* k of WB_DIR / WB_RESQ, 1..8 (the pages evaluate 2, 3, 4); 0 otherwise */
    int32_t budget;            /* WB_BUDGET_HEAD or WB_BUDGET_LAYER (BITALLOC, H * dk <= 4096); 0 otherwise */
    int32_t int_bits;          /* HAD_INT8 / MIXED integer tier ([DAMP] "Quantization & calibration
                                * details"): 0 or 8 for INT8, 4 for INT4 (codes two a byte, low nibble
                                * first, 15 affine steps); 0 for the other layouts */
    uint64_t seed;             /* Philox key for WB_SR */
} wb_layout_desc;

typedef struct wb_state wb_state;   /* opaque host-side handle */

/* Device bytes needed for the state buffer and for the side buffer of the auxiliary
 * write-back state -- float32 per element: the error-feedback residual (WB_EF), the
 * k-bit residual's value (WB_RESQ) or the direction counter (WB_DIR); 0 for the other
 * rules and for FP32. Host only. */
int state_bytes(const wb_layout_desc* d, size_t* state_bytes_out, size_t* side_bytes_out);

/* Bind a handle to caller-owned device memory and write the zero state S_0 = 0 with
 * e_0 = 0 ([WB-zh] "Reproduction assessment": auxiliary write-back state reset).
 * BITALLOC rows start at width bbar with k = 15 (f = 1). `perm` (MIXED only; NULL
 * otherwise) is a host array uint8 [H][dk], each row a permutation of 0..dk-1, copied
 * into the state buffer ([DAMP] "Implementation": a static per-head permutation
 * places the protected rows contiguously). The handle is host memory owned by the
 * library until state_free. */
int state_alloc(const wb_layout_desc* d, void* dev_state, size_t state_bytes,
                void* dev_side, size_t side_bytes, const uint8_t* perm,
                void* stream, wb_state** out);

/* Release the handle; never the caller's buffers. */
int state_free(wb_state* st);

/* One decode token with write-back (cadence C = 1). For every head: dequantize the
 * stored state, apply S_t = (I - beta k k^T) Diag(e^{-s}) S_{t-1} + beta k v^T,
 * write o_t = S_t^T q_t taken before quantization, then requantize S_t under the
 * handle's rule and store it in place ([LBRS] "Accumulated readout error"; [DAMP]
 * "Implementation": reconstruct, update, re-quantize, write back). `t` is the token
 * index that keys stochastic rounding. */
int state_step_decode(wb_state* st, const float* q, const float* k, const float* v,
                      const float* beta, const float* s, float* o, uint64_t t, void* stream);

/* Prefill T tokens with deferred write-back ([LBRS] "Accumulated readout error": write
 * back every C tokens, per prefill chunk, or deferred with C = 8). q, k, v are
 * bfloat16 bit patterns [B][T][H][d]; beta float32 [B][T][H]; s float32 [B][T][H][dk]
 * or [B][T][H]; o float32 [B][T][H][dv]. The state is written back after tokens
 * t0 + i with (i + 1) % C == 0 and after the last token; outputs come from the
 * unquantized running state. The call is evaluated in segments that end at every
 * write-back point and are at most min(chunk, 8) tokens long (chunk >= 1, EINVAL
 * otherwise; the result does not depend on it: the recurrence is exact between
 * write-backs). The state path runs in float64. Supported: FP32, UNIFORM, HAD_INT8 and
 * MIXED (k_hi = 16) with 32-value blocks and 8-bit codes, round to nearest, dk = dv =
 * 128 (EUNSUPPORTED otherwise). */
int state_prefill_chunk(wb_state* st, const uint16_t* q_bf16, const uint16_t* k_bf16,
                        const uint16_t* v_bf16, const float* beta, const float* s, float* o,
                        int T, int chunk, int C, uint64_t t0, void* stream);

/* UNIFORM only: write-activity diagnostics ([WB] "Methods": "Direction-memory events",
 * "Persistence metrics", "State diagnostics"; "Write-back behavior"). `dev_counters`
 * (uint32 [B*H][8]) and `dev_votes` (uint8 [B*H][dk][dv], one byte per element) are
 * device buffers, 16-byte aligned, caller-owned and zeroed by the caller at the start
 * of a sequence; both non-NULL or both NULL (EINVAL otherwise; NULL stops counting).
 * With q the level entering a decode step, h the updated value, delta = h - q and
 * M = 2 |delta| / step, every following decode step adds per head:
 *   [0] elements with M < 1 (the dead zone);
 *   [1] elements whose stored level changed;
 *   [2] eligible votes, step/8 < |delta| < step/2 (under every rule);
 *   [3] direction-memory triggers (WB_DIR; a trigger at a rail moves nothing);
 *   [4] sub-threshold writes: M < 1 and the level changed;
 *   [5] / [6] votes following a vote of the same / the other sign on the previous step;
 *   [7] runs started: votes that do not continue a run of same-sign votes on
 *       consecutive steps (a run ends at a reversal, a step without a vote, or a vote
 *       step that changed the level or triggered). Mean run length = [2] / [7].
 * `dev_votes` carries, per element, the previous step's vote: 0 none, 1 / 2 a
 * positive / negative vote whose run is open, 5 / 6 one whose run closed. Prefill
 * write-backs neither count nor update it. */
int state_set_activity(wb_state* st, uint32_t* dev_counters, uint8_t* dev_votes);

/* BITALLOC, RTN or SR: one decode token (inputs as state_step_decode) whose write-back
 * first allocates ([LBRS] "State bit allocation": widths are set at each write-back,
 * at the state's budget, per head or layer-wise; "Levels and storage"): the step runs
 * from the stored state, the token is folded into the attached estimators (if any),
 * then widths, clipping fits and Delta_i are chosen as in state_allocate_bits but for
 * the updated state S_t itself, and S_t is rounded once onto the new grid: to nearest
 * (RTN) or stochastically with the Philox draws of token t (SR, as state_step_decode).
 * Layer-wise budget: the widths of a sequence's rows come from all its H heads, so the
 * call runs three launches on `stream` (costs of every head's updated state, the
 * widths per sequence, then the step once more with the fits and the rounding); the
 * workspace is the state's own. The allocation takes s_i and r_i from the estimators
 * when attached, else this token's decays and r_i = 1/(3 dk). o as in
 * state_step_decode. EUNSUPPORTED for other layouts and for EF. */
int state_step_decode_alloc(wb_state* st, const float* q, const float* k, const float* v, const float* beta,
                            const float* s, float* o, uint64_t t, int factor, int C, void* stream);

/* BITALLOC only: online estimators of the decay and erasure terms ([LBRS] "State bit
 * allocation"). `dev_est` (float32 [B*H][2 dk + 4], 16-byte aligned, caller-owned,
 * zeroed by the caller at the start of a sequence; NULL detaches) holds per head the
 * unnormalised span-64 exponential averages (alpha = 2/65 per token) N_a[dk] of
 * 1 - e^{-2 s_i} and N_r[dk] of beta (2 - beta) k_i^2, then their weight sum W (and
 * three unused floats). Every following decode step folds its token in:
 * N <- (1 - alpha) N + alpha x, W <- (1 - alpha) W + alpha. The estimates are
 * s_i = -1/2 log1p(-N_a / W) and r_i = N_r / (2 W). */
int state_set_estimators(wb_state* st, float* dev_est);

/* BITALLOC only: recompute per-row widths and clipping-fit indices from the stored
 * state and repack it in place ([LBRS] "Approximate erasure rate", "Range
 * normalization", "State bit allocation", "Choice of persistence factor", "Levels and
 * storage"; [LBRS-x]): R_i = row max |S|, R~_i = R_i / RMS_j R_j, Gamma_i the
 * persistence factor `factor` (WB_GAMMA_*) at cadence C >= 1, c_i = Gamma_i R~_i^2 kept
 * in [1e-300, 1e300], b_i = bbar + 0.5 log2(c_i / geomean(c)) rounded (ties even),
 * clipped to [bmin, bmax], adjusted greedily to sum = bbar*dk; f fitted over
 * 1/4 + k/20 by squared error. s, r: float32 [B][H][dk]; r may be NULL for
 * r_i = 1/(3 dk) (E[beta(2-beta)] = 2/3, E[k_i^2] = 1/dk for the synthetic stream).
 * s NULL (then r must be NULL): s_i and r_i from the attached estimators; a head whose
 * estimators have seen no token (W = 0) gives every row Gamma = 1. EINVAL for a bad
 * factor, C < 1, or s NULL without estimators. */
int state_allocate_bits(wb_state* st, const float* s, const float* r, int factor, int C, void* stream);

/* For callers that cannot allocate device memory or must not touch the state buffer's
 * workspace (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): state_allocate_bits with the same arguments and results, whose
 * workspace (layer-wise budget and HEADALLOC: a float64 cost and a uint8 width per row
 * of the layer, 9 * B * H * dk bytes, HEADALLOC 9 * B * H) is a static device array of
 * the library, 16 MiB per GPU (B * H <= 14563 heads at dk = 128 under the layer
 * budget), held by each GPU the library runs on until the process ends. Nothing is
 * allocated, by the library or by any routine it calls. WB_ESCRATCH if the workspace
 * exceeds the array; WB_ELAUNCH if its device address could not be found when the
 * handle was made. Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (several streams, several threads) race and must be ordered by
 * the caller. A per-head budget uses no workspace and runs as state_allocate_bits. */
int state_allocate_bits_static(wb_state* st, const float* s, const float* r, int factor, int C, void* stream);

/* Export: the stored state dequantized to float32 S [B][H][dk][dv] in the original
 * domain and logical row order (Hadamard rows rotated back, rows un-permuted). */
int state_dequant(const wb_state* st, float* S, void* stream);

/* Import: one round-to-nearest write-back of the float32 state S [B][H][dk][dv]
 * (logical order); BITALLOC keeps its current widths and fit indices; the
 * error-feedback residuals are reset to 0. */
int state_quantize(wb_state* st, const float* S, void* stream);

/* Raw device pointers of the stored bytes and side buffer (for checkpoints and
 * byte-exact comparison). Host only. */
int state_export(const wb_state* st, void** dev_state, size_t* bytes, void** dev_side);

/* DAMP calibration ([DAMP] "Risk scoring and selection", "Quantization & calibration
 * details"): from N sampled unquantized states `samples` float32 [N][H][dk][dv]
 * (logical order) and decay rates s float32 [H][dk], compute per head and row
 * E_u = mean ||x_u - H deQ(Q(H x_u))||^2 (affine INT8 blocks of `block` values, nearest
 * rounding), P_u = 1/max(1 - e^{-2 s_u}, tau), C_u = E_u P_u; write the costs to
 * cost_out float32 [H][dk] (may be NULL) and the permutation to perm_out uint8
 * [H][dk]: the k_hi highest-cost rows (ties to the lower index) in ascending order,
 * then the rest in ascending order. dv = 128, dk = 128. */
int state_damp_select(const float* samples, int N, int H, int dk, int dv, int block, int k_hi,
                      const float* s, float tau, float* cost_out, uint8_t* perm_out,
                      void* stream);

/* Text of a status code. */
const char* state_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* WBSTATE_H */
