// Decay-aware per-row bit allocation pass (BITALLOC layout), one workgroup per head.
//
// [LBRS] "Approximate erasure rate", "Range normalization", "State bit allocation",
// "Levels and storage"; [LBRS-x] (cost c = Gamma-hat * R~^2 and the width rule):
//   R_i   = max_j |S_ij| of the stored state;  R~_i = R_i / RMS_j R_j (one head);
//   Gamma = the persistence factor ([LBRS] "Choice of persistence factor"): by default
//   1 / (C expm1(2 (s_i + r_i))), else 1 / (1 - e^{-2 s_i}) (DAMP's, uncapped) or
//   1 / (1 - e^{-2 C s_i}); s_i, r_i given, or from the online estimators
//   (s = -1/2 log1p(-N_a / W), r = N_r / (2 W); W = 0: Gamma = 1 for every row);
//   c_i = Gamma R~_i^2 kept in [1e-300, 1e300];
//   b*_i  = bbar + 0.5 log2(c_i / GM(c));  b_i = clip(rint(b*_i), bmin, bmax), then one
//   bit at a time: while short, +1 to the largest (3/4) c 2^{-2b} among b < bmax; while
//   over, -1 to the smallest 3 c 2^{-2b} among b > bmin; ties to the lower row;
//   all R_i = 0 keeps every row at bbar;
//   fit: f_k = 1/4 + k/20, Delta_k = f16(f_k R_i / n_i), the smallest squared rounding
//   error wins, ties to the larger f;
//   repack: the stored values rounded to nearest on the new grid, new prefix offsets.
// Widths are decided in float64. The stored values are exact in float32 (|kappa| <=
// 127 times a float16 step), the 16 candidate steps per row come from float64 exactly
// as defined, and the candidates' squared errors are summed in float32: an element
// whose rounding is a near-tie contributes (almost) the same error either way, so
// only errors within ~1e-7 of each other can be ordered differently. The rounding that
// is stored (the repack) is exact: float32 where the quotient is clear of a
// half-integer, float64 division otherwise.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256, NCG = 16, RS = 16;
constexpr float kMagic = 12582912.0f;          // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

// fit fractions f_k = 1/4 + k/20 in float64 (the same operations, at compile time)
struct FitTable {
    double f[16];
    constexpr FitTable() : f() {
        for (int k = 0; k < 16; ++k) f[k] = 0.25 + k / 20.0;
    }
};
__constant__ FitTable kFit = FitTable();

struct AllocSmem {
    uint32_t reg[(DK * DV + 3 * DK) / 4 + 4];
    int width[DK], fit[DK], off[DK], newoff[DK];
    float delta[DK];
    double R[DK], c[DK];
    float2 cand[DK][16];                       // (Delta_k, 1 / Delta_k) per row and fit index
    int order[DK];                             // rows by increasing stored width
    int newwidth[DK];
    int newfit[DK];
    uint16_t newdelta[DK];
};

// persistence factor of one row (WB_GAMMA_*); an infinite value is capped by the caller
__device__ __forceinline__ double persistence(int factor, int C, double s, double r) {
    if (factor == WB_GAMMA_W1) return 1.0 / -expm1(-2.0 * s);
    if (factor == WB_GAMMA_HC) return 1.0 / -expm1(-2.0 * double(C) * s);
    return 1.0 / (double(C) * expm1(2.0 * (s + r)));
}

// sum over the 16 lanes of a DPP row (the 16 column groups of one state row)
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // xor 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // xor 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // mirror
    return v;
}

// one step of a (smallest error, then largest fit index) reduction over a DPP row
template <int CTRL>
__device__ __forceinline__ void argmin_step(float& be, int& best) {
    const float oe = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(be), CTRL, 0xF, 0xF, false));
    const int ob = __builtin_amdgcn_update_dpp(0, best, CTRL, 0xF, 0xF, false);
    const bool take = oe < be || (oe == be && ob > best);
    be = take ? oe : be;
    best = take ? ob : best;
}

// Clipping fit of one row from level counts. The row's stored values lie on its old
// grid (kappa Delta_old) and a value's rounding error depends only on a = |kappa| <=
// n_old < 16 NWD: each lane counts the levels of its 8 values in 4-bit fields (NWD
// 64-bit words), the counts are widened to 8-bit fields and summed over the row's 16
// lanes, lane cg evaluates fit index cg (step dk.x, reciprocal dk.y, levels clamped to
// [lo, hi] in magic-number form) as a sum over the levels, and the row's smallest error
// (ties to the larger f) is found over the 16 lanes.
template <int NWD>
__device__ __forceinline__ int level_fit(const float x[8], float dl, int nold, float2 dk, float lo, float hi,
                                         int cg) {
    const float inv4 = dl > 0.f ? 4.f / dl : 0.f;
    uint64_t h[NWD];
#pragma unroll
    for (int w = 0; w < NWD; ++w) h[w] = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t a4 = uint32_t(__builtin_fmaf(fabsf(x[c]), inv4, 0.5f));     // 4 a
        const uint64_t one = 1ull << (a4 & 63);
        if constexpr (NWD == 1) {
            h[0] += one;
        } else {
            h[0] += a4 < 64 ? one : 0ull;
            h[1] += a4 < 64 ? 0ull : one;
        }
    }
    // cnt[4 w + 0]: levels 16 w + 0, 2, 4, 6; + 1: 1, 3, 5, 7; + 2: 8, 10, ..; + 3: 9, 11, ..
    uint32_t cnt[4 * NWD];
#pragma unroll
    for (int w = 0; w < NWD; ++w) {
        cnt[4 * w + 0] = uint32_t(h[w]) & 0x0F0F0F0Fu;
        cnt[4 * w + 1] = uint32_t(h[w] >> 4) & 0x0F0F0F0Fu;
        cnt[4 * w + 2] = uint32_t(h[w] >> 32) & 0x0F0F0F0Fu;
        cnt[4 * w + 3] = uint32_t(h[w] >> 36) & 0x0F0F0F0Fu;
    }
#pragma unroll
    for (int i = 0; i < 4 * NWD; ++i) {
        cnt[i] += uint32_t(__builtin_amdgcn_update_dpp(0, int(cnt[i]), 0xB1, 0xF, 0xF, false));
        cnt[i] += uint32_t(__builtin_amdgcn_update_dpp(0, int(cnt[i]), 0x4E, 0xF, 0xF, false));
        cnt[i] += uint32_t(__builtin_amdgcn_update_dpp(0, int(cnt[i]), 0x141, 0xF, 0xF, false));
        cnt[i] += uint32_t(__builtin_amdgcn_update_dpp(0, int(cnt[i]), 0x140, 0xF, 0xF, false));
    }
    float e = 0.f;
#pragma unroll
    for (int a = 1; a < 16 * NWD; ++a) {
        if (a <= nold) {
            const int l = a & 15;
            const uint32_t word = cnt[4 * (a >> 4) + (l & 1) + 2 * (l >> 3)];
            const float ca = float((word >> (8 * ((l >> 1) & 3))) & 255u);
            const float xa = float(a) * dl;                                  // exact
            const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(xa, dk.y, kMagic), lo, hi);
            const float r = __builtin_fmaf(-dk.x, y - kMagic, xa);
            e = __builtin_fmaf(ca * r, r, e);
        }
    }
    float be = e;
    int best = cg;
    argmin_step<0xB1>(be, best);
    argmin_step<0x4E>(be, best);
    argmin_step<0x141>(be, best);
    argmin_step<0x140>(be, best);
    return best;
}

// number of set bits of a wavefront mask below the calling lane
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// STEP = false: the allocation pass on the stored state. STEP = true: one decode token
// whose write-back allocates: the stored state is dequantized, the delta-rule step
// (u = k^T D S, w = beta (v - u), S' = D S + k w^T, o = S'^T q) runs in float32, the
// token is folded into the estimators, and the widths, fits and codes are chosen
// for S' (every row through the 16-candidate fit: S' is not on the old grid).
enum { kHead = 0, kStep = 1, kCost = 2, kPack = 3, kStepCost = 4, kStepPack = 5 };

// MODE kHead: the allocation pass on the stored state (per-head budget). kStep: one
// decode token whose write-back allocates (see below). Layer-wise budget: kCost writes
// each row's cost c_i (0 for a head whose rows are all zero) to the workspace and
// stops; kPack takes the widths the per-sequence pass left in the workspace, then
// fits and repacks as kHead does. kStepCost / kStepPack are the same two halves for a
// decode token whose write-back allocates under the layer budget: both run the token's
// step from the stored state (the same operations, so the same updated state), the
// first writes the outputs, folds the token into the estimators and leaves the costs
// of the updated state, the second fits and rounds it at the widths of the layer.
// OB: rows may be one bit wide (bmin = 1); without it that path is not compiled.
// SR: the allocating write-back rounds stochastically (Philox draws of the element:
// row, column group of 8, head, token), as the decode write-back does.
template <int MODE, bool OB, bool SR>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) allocate_kernel(const AllocArgs A) {
    constexpr bool STEP = MODE == kStep || MODE == kStepCost || MODE == kStepPack;
    constexpr bool COST = MODE == kCost || MODE == kStepCost;
    constexpr bool PACK = MODE == kPack || MODE == kStepPack;
    static_assert(STEP || !SR, "stochastic rounding is a rule of the decode write-back");
    __shared__ AllocSmem sm;
    // decode-step scratch, in the candidate table (filled only after the step)
    float* const fk = reinterpret_cast<float*>(&sm.cand[0][0]);
    float* const fq = fk + DK;
    float* const fa = fq + DK;
    float* const red = fa + DK;                   // [4 wavefronts][DV]
    static_assert(sizeof(sm.cand) >= sizeof(float) * (3 * DK + 4 * DV), "step scratch");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int head = blockIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int code_bytes = A.code_cap;         // Delta and meta follow the code area
    const int total = code_bytes + 3 * DK;

    // the region straight into LDS (global-to-LDS loads, all issued at once): vectors
    // i0 + lane, i0 = 64 wave + 256 r (a scalar)
    for (int i0 = 64 * wave; i0 * 16 < total; i0 += NT)
        if ((i0 + lane) * 16 < total) lds_load16(reinterpret_cast<const uint4*>(region) + i0 + lane, &sm.reg[4 * i0]);
    if constexpr (STEP) {
        if (tid < DK) {
            const size_t rb = (size_t)head * DK + tid;
            const float sv = A.s_per_row ? A.sd[rb] : A.sd[head];
            fk[tid] = A.k[rb];
            fq[tid] = A.q[rb];
            fa[tid] = expf(-sv);
            if (MODE != kStepPack && A.est)
                ema_fold_row(A.est + (size_t)head * est_stride(DK), DK, tid, sv, A.beta[head], fk[tid]);
        }
    }
    lds_loads_wait();
    __syncthreads();
    const uint8_t* bytes = reinterpret_cast<const uint8_t*>(sm.reg);
    if (wave == 0) {
        // (the rest of the workgroup waits for this wavefront: raised issue priority)
        __builtin_amdgcn_s_setprio(3);
        int wv[2], local = 0;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 2 * lane + r;
            const int meta = bytes[code_bytes + 2 * DK + row];
            const int wdt = (meta & 7) + 1;
            sm.width[row] = wdt;
            sm.fit[row] = meta >> 4;
            sm.delta[row] = f16_bits_to_f32(uint32_t(bytes[code_bytes + 2 * row]) |
                                            (uint32_t(bytes[code_bytes + 2 * row + 1]) << 8));
            wv[r] = wdt * (DV / 8);
            local += wv[r];
        }
        int incl = local;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        sm.off[2 * lane] = incl - local;
        sm.off[2 * lane + 1] = incl - local + wv[0];
        // rank of rows 2 lane and 2 lane + 1 in (stored width, row) order (ballots)
        const int w0 = wv[0] / (DV / 8), w1 = wv[1] / (DV / 8);
        int before = 0, pos0 = 0, pos1 = 0;
#pragma unroll
        for (int v = 1; v <= 8; ++v) {
            const unsigned long long m0 = __ballot(w0 == v), m1 = __ballot(w1 == v);
            const int below = lanes_below(m0) + lanes_below(m1);
            if (w0 == v) pos0 = before + below;
            if (w1 == v) pos1 = before + below + int(w0 == v);
            before += __popcll(m0) + __popcll(m1);
        }
        sm.order[pos0] = 2 * lane;
        sm.order[pos1] = 2 * lane + 1;
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();

    // stored values (exact in float32: |kappa| <= 127 times a float16 Delta); the rows
    // are visited in stored-width order, so the 4 rows of a wavefront step nearly
    // always share a width
    float x[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int row = sm.order[rg + RS * m];
        const int bw = sm.width[row];
        const int n = (1 << (bw - 1)) - 1;
        const int off = sm.off[row] + cg * bw;
        const int wi = off >> 2, sh = (off & 3) * 8;
        uint64_t fld = (uint64_t(sm.reg[wi]) | (uint64_t(sm.reg[wi + 1]) << 32)) >> sh;
        if (sh) fld |= uint64_t(sm.reg[wi + 2]) << (64 - sh);
        const float dl = sm.delta[row];
        float R = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int field = int((fld >> (c * bw)) & ((1ull << bw) - 1));
            const int kap = (OB && bw == 1) ? 2 * field - 1 : field - n;    // one-bit rows: -1, +1
            x[m][c] = float(kap) * dl;
            R = fmaxf(R, fabsf(x[m][c]));
        }
        if constexpr (!STEP) {
            // maximum over the row's 16 lanes (a DPP row; non-negative values)
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0xB1, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x4E, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x141, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x140, 0xF, 0xF, false)));
            if (cg == 0) sm.R[row] = double(R);
        }
    }
    if constexpr (STEP) {
        // u_j = sum_i k_i a_i S_ij: this thread's 8 rows, then the 4 row groups of the
        // wavefront (lanes 16 and 32 apart), then the 4 wavefronts through LDS
        float u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = sm.order[rg + RS * m];
            const float ka = fk[row] * fa[row];
#pragma unroll
            for (int c = 0; c < 8; ++c) u[c] = __builtin_fmaf(ka, x[m][c], u[c]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) u[c] = add_xor32_f32(add_xor16_f32(u[c]));
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) red[wave * DV + 8 * cg + c] = u[c];
        }
        __syncthreads();
        const float beta = A.beta[head];
        float w[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int col = 8 * cg + c;
            const float uj = (red[col] + red[DV + col]) + (red[2 * DV + col] + red[3 * DV + col]);
            w[c] = beta * (A.v[(size_t)head * DV + col] - uj);
        }
        __syncthreads();
        // S' = D S + k w^T and o_j = sum_i q_i S'_ij
        float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = sm.order[rg + RS * m];
            const float a = fa[row], kk = fk[row], qq = fq[row];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                x[m][c] = __builtin_fmaf(kk, w[c], a * x[m][c]);
                p[c] = __builtin_fmaf(qq, x[m][c], p[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) p[c] = add_xor32_f32(add_xor16_f32(p[c]));
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) red[wave * DV + 8 * cg + c] = p[c];
        }
        __syncthreads();
        if (MODE != kStepPack && tid < DV)
            A.o[(size_t)head * DV + tid] = (red[tid] + red[DV + tid]) + (red[2 * DV + tid] + red[3 * DV + tid]);
    }
    if constexpr (STEP) {
        // row maxima of the updated state, over the row's 16 lanes (a DPP row)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            float R = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) R = fmaxf(R, fabsf(x[m][c]));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0xB1, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x4E, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x141, 0xF, 0xF, false)));
            R = fmaxf(R, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(R), 0x140, 0xF, 0xF, false)));
            if (cg == 0) sm.R[sm.order[rg + RS * m]] = double(R);
        }
    }
    __syncthreads();

    // widths (one wavefront, at raised issue priority; lane l owns rows 2l and 2l+1)
    if (wave == 0) {
        __builtin_amdgcn_s_setprio(3);
        const int r0 = 2 * lane, r1 = r0 + 1;
        const double R0 = sm.R[r0], R1 = sm.R[r1];
        // (the squares of float32 maxima cannot underflow in float64: some R > 0 iff sq > 0)
        const double sq = wave_sum_f64<1>(R0 * R0 + R1 * R1);
        int b0 = A.bbar, b1 = A.bbar;
        double c0 = 0.0, c1 = 0.0;
        if (!PACK && sq > 0.0) {
            const double rms = sqrt(sq / double(DK));
            const size_t base = (size_t)head * DK;
            double s0, s1, q0, q1;
            bool flat = false;
            if (A.s) {
                s0 = A.s[base + r0];
                s1 = A.s[base + r1];
                q0 = A.r ? double(A.r[base + r0]) : double(A.r_default);
                q1 = A.r ? double(A.r[base + r1]) : double(A.r_default);
            } else if (STEP && !A.est) {
                // the decode token's own decays
                s0 = A.s_per_row ? A.sd[base + r0] : A.sd[head];
                s1 = A.s_per_row ? A.sd[base + r1] : A.sd[head];
                q0 = q1 = double(A.r_default);
            } else {
                const float* e = A.est + (size_t)head * est_stride(DK);
                const double W = e[2 * DK];
                flat = !(W > 0.0);
                s0 = -0.5 * log1p(-double(e[r0]) / W);
                s1 = -0.5 * log1p(-double(e[r1]) / W);
                q0 = 0.5 * double(e[DK + r0]) / W;
                q1 = 0.5 * double(e[DK + r1]) / W;
            }
            const double g0 = flat ? 1.0 : persistence(A.factor, A.cadence, s0, q0);
            const double g1 = flat ? 1.0 : persistence(A.factor, A.cadence, s1, q1);
            const double rt0 = R0 / rms, rt1 = R1 / rms;
            c0 = fmin(fmax(g0 * (rt0 * rt0), 1e-300), 1e300);
            c1 = fmin(fmax(g1 * (rt1 * rt1), 1e-300), 1e300);
            if constexpr (COST) {
                A.ws_c[base + r0] = c0;
                A.ws_c[base + r1] = c1;
            } else {
            const double lsum = wave_sum_f64<1>(log(c0) + log(c1));
            const double gm = exp(lsum / double(DK));
            const double bs0 = double(A.bbar) + 0.5 * log2(c0 / gm);
            const double bs1 = double(A.bbar) + 0.5 * log2(c1 / gm);
            b0 = int(fmin(fmax(rint(bs0), double(A.bmin)), double(A.bmax)));
            b1 = int(fmin(fmax(rint(bs1), double(A.bmin)), double(A.bmax)));
            const int target = A.bbar * DK;
            const int tot = int(wave_sum_f64<1>(double(b0 + b1)));      // exact: small integers
            // One bit at a time toward the budget, each time to the row of largest gain
            // (3/4) c 2^{-2b} (b < bmax) or, when over, from the row of smallest loss
            // 3 c 2^{-2b} (b > bmin), ties to the lower row. A row's successive gains
            // shrink by exactly 1/4 (losses grow by 4), so the moves made are the
            // `moves` first candidates (row, step) in the order (value, then row): with
            // an order-preserving 64-bit key per candidate (the value's bits for gains,
            // their complement for losses), the key of the last move made is found by a
            // bitwise search on the count of keys at or above it (ballots) -- first on
            // the high 32 bits, then on the low 32 bits of the keys that share the high
            // word found (skipped when only one does) -- and of the candidates equal to it
            // the lowest rows are taken.
            const bool grow = tot < target;
            const int moves = grow ? target - tot : tot - target;
            if (moves > 0) {
                constexpr int MS = 6;                         // bmax - bmin <= 6
                const int lim0 = grow ? A.bmax - b0 : b0 - A.bmin;
                const int lim1 = grow ? A.bmax - b1 : b1 - A.bmin;
                double v0 = grow ? (0.75 * c0) * exp2(-2.0 * b0) : (3.0 * c0) * exp2(-2.0 * b0);
                double v1 = grow ? (0.75 * c1) * exp2(-2.0 * b1) : (3.0 * c1) * exp2(-2.0 * b1);
                const double scale = grow ? 0.25 : 4.0;
                uint64_t key0[MS], key1[MS];                  // 0: no such candidate
#pragma unroll
                for (int st = 0; st < MS; ++st) {
                    const uint64_t r0b = uint64_t(__double_as_longlong(v0)), r1b = uint64_t(__double_as_longlong(v1));
                    key0[st] = st < lim0 ? (grow ? r0b : ~r0b) : 0ull;
                    key1[st] = st < lim1 ? (grow ? r1b : ~r1b) : 0ull;
                    v0 *= scale;
                    v1 *= scale;
                }
                auto count_gt = [&](uint64_t t) {
                    int cnt = 0;
#pragma unroll
                    for (int st = 0; st < MS; ++st)
                        cnt += __popcll(__ballot(key0[st] > t)) + __popcll(__ballot(key1[st] > t));
                    return cnt;
                };
                // high word: the largest H with at least `moves` keys whose high word >= H
                uint32_t H = 0;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t cand = H | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int st = 0; st < MS; ++st)
                        cnt += __popcll(__ballot(uint32_t(key0[st] >> 32) >= cand)) +
                               __popcll(__ballot(uint32_t(key1[st] >> 32) >= cand));
                    if (cnt >= moves) H = cand;
                }
                // keys with high word H: `need` of them are taken, the largest low words
                const int need = moves - count_gt((uint64_t(H) << 32) | 0xFFFFFFFFull);
                int neq = 0;
                uint32_t L = 0;
#pragma unroll
                for (int st = 0; st < MS; ++st) {
                    const unsigned long long e0 = __ballot(uint32_t(key0[st] >> 32) == H);
                    const unsigned long long e1 = __ballot(uint32_t(key1[st] >> 32) == H);
                    neq += __popcll(e0) + __popcll(e1);
                    // (the low word of one of them, kept when it is the only one)
                    if (e0) L = __builtin_amdgcn_readlane(uint32_t(key0[st]), __builtin_ctzll(e0));
                    if (e1) L = __builtin_amdgcn_readlane(uint32_t(key1[st]), __builtin_ctzll(e1));
                }
                if (neq > 1) {
                    L = 0;
                    for (int bit = 31; bit >= 0; --bit) {
                        const uint32_t cand = L | (1u << bit);
                        int cnt = 0;
#pragma unroll
                        for (int st = 0; st < MS; ++st)
                            cnt += __popcll(__ballot(uint32_t(key0[st] >> 32) == H && uint32_t(key0[st]) >= cand)) +
                                   __popcll(__ballot(uint32_t(key1[st] >> 32) == H && uint32_t(key1[st]) >= cand));
                        if (cnt >= need) L = cand;
                    }
                }
                const uint64_t T = (uint64_t(H) << 32) | L;   // the key of the last move
                const int rem = moves - count_gt(T);          // equal keys still to take
                int a0 = 0, a1 = 0;
                bool t0 = false, t1 = false;
#pragma unroll
                for (int st = 0; st < MS; ++st) {
                    a0 += key0[st] > T;
                    a1 += key1[st] > T;
                    t0 |= key0[st] == T;
                    t1 |= key1[st] == T;
                }
                // rank of each tied row among the tied rows (rows 2 lane, 2 lane + 1)
                const int below = lanes_below(__ballot(t0)) + lanes_below(__ballot(t1));
                if (t0 && below < rem) ++a0;
                if (t1 && below + int(t0) < rem) ++a1;
                b0 += grow ? a0 : -a0;
                b1 += grow ? a1 : -a1;
            }
            }
        } else if constexpr (COST) {
            A.ws_c[(size_t)head * DK + r0] = 0.0;        // a head whose rows are all zero
            A.ws_c[(size_t)head * DK + r1] = 0.0;
        }
        if constexpr (PACK) {
            b0 = A.ws_w[(size_t)head * DK + r0];
            b1 = A.ws_w[(size_t)head * DK + r1];
        }
        sm.newwidth[r0] = b0;
        sm.newwidth[r1] = b1;
        int local = (b0 + b1) * (DV / 8);
        int incl = local;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        sm.newoff[r0] = incl - local;
        sm.newoff[r1] = incl - local + b0 * (DV / 8);
        __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (COST) return;
    __syncthreads();

    // candidate steps: thread t fills fit index t % 16 of rows t / 16 + 16 m
    for (int i = tid; i < DK * 16; i += NT) {
        const int row = i >> 4, kf = i & 15;
        const int n = (1 << (sm.newwidth[row] - 1)) - 1;      // 0: a one-bit row, no fit
        const float d = n ? f16_bits_to_f32(f64_to_f16_bits(kFit.f[kf] * sm.R[row] / n)) : 0.f;
        // reciprocal refined by one Newton step: it only orders candidate errors and
        // pre-rounds the repack, which falls back to an exact quotient near half-integers
        float r = __builtin_amdgcn_rcpf(d);
        r = __builtin_fmaf(__builtin_fmaf(-d, r, 1.f), r, r);
        sm.cand[row][kf] = make_float2(d, d > 0.f ? r : 0.f);
    }
    // clipping fit and repack
    for (int i = tid; i < code_bytes / 4; i += NT) sm.reg[i] = 0u;
    __syncthreads();
#pragma clang loop unroll(full)
    for (int m = 0; m < 8; ++m) {
        const int row = sm.order[rg + RS * m];
        const int bw = sm.newwidth[row];
        const int n = (1 << (bw - 1)) - 1;
        const float lo = kMagic - float(n), hi = kMagic + float(n);
        const int bwo = sm.width[row];
        const int nold = (OB && bwo == 1) ? 1 : (1 << (bwo - 1)) - 1;    // one-bit rows hold levels -1, +1
        int best = 15;
        uint16_t dbits = 0;
        uint64_t fld = 0;
        uint32_t r16[8];
        if constexpr (SR) sr_draws8(A.seed, uint32_t(head), A.t, row, cg, r16);
        if (OB && bw == 1) {
            // one-bit row ([LBRS] "Levels and storage"): Delta = f16(mean |x|), the sign
            // (nearest of -Delta, +Delta: an exact zero is the tie and takes -Delta); the
            // sum is exact in float64 for values on the old grid
            double sa = 0.0;
#pragma unroll
            for (int c = 0; c < 8; ++c) sa += fabs(double(x[m][c]));
            sa += dpp_f64<0xB1>(sa);
            sa += dpp_f64<0x4E>(sa);
            sa += dpp_f64<0x141>(sa);
            sa += dpp_f64<0x140>(sa);
            dbits = f64_to_f16_bits(sa / double(DV));
            if (dbits) {
                if constexpr (SR) {
                    // the levels -Delta + k 2 Delta, k = floor(tau) + [u < frac(tau)],
                    // tau = (x + Delta) / (2 Delta), clamped to [0, 1]
                    const float d = f16_bits_to_f32(dbits);
                    const float h = 0.5f / d;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float tau = __builtin_fmaf(x[m][c], h, 0.5f);
                        const float fl = floorf(tau);
                        const float k = fminf(fmaxf(fl + ((float(r16[c]) < (tau - fl) * 65536.f) ? 1.f : 0.f), 0.f), 1.f);
                        fld |= uint64_t(k > 0.f) << c;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) fld |= uint64_t(x[m][c] > 0.f) << c;
                }
            }
        } else {
        if (!STEP && bwo <= 5) {
            best = level_fit<1>(x[m], sm.delta[row], nold, sm.cand[row][cg], lo, hi, cg);
        } else if (!STEP && bwo == 6) {
            best = level_fit<2>(x[m], sm.delta[row], nold, sm.cand[row][cg], lo, hi, cg);
        } else {
            float err[16];
#pragma unroll
            for (int kf = 0; kf < 16; ++kf) {
                const float2 dk = sm.cand[row][kf];
                float e = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float y = __builtin_amdgcn_fmed3f(__builtin_fmaf(x[m][c], dk.y, kMagic), lo, hi);
                    const float r = __builtin_fmaf(-dk.x, y - kMagic, x[m][c]);
                    e = __builtin_fmaf(r, r, e);
                }
                err[kf] = row16_sum(e);
            }
            best = 15;
            float be = err[15];
#pragma unroll
            for (int kf = 14; kf >= 0; --kf)     // ties go to the larger f
                if (err[kf] < be) {
                    be = err[kf];
                    best = kf;
                }
        }
        const float2 dk = sm.cand[row][best];
        dbits = f32_to_f16_bits(dk.x);
        if constexpr (SR) {
            // floor(tau) + [u < frac(tau)] with tau = x / Delta and u the element's 16-bit
            // draw over 2^16, clamped to [-n, n]; a zero step stores level 0
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float tau = x[m][c] * dk.y;
                const float fl = floorf(tau);
                const float k = fminf(fmaxf(fl + ((float(r16[c]) < (tau - fl) * 65536.f) ? 1.f : 0.f), -float(n)),
                                      float(n));
                fld |= uint64_t(uint32_t(int(k) + n)) << (c * bw);
            }
        } else
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // nearest level, ties to even, of the exact quotient x / Delta: x / Delta +
            // 1.5 * 2^23 rounded once (its fraction, x / Delta - level, one more FMA);
            // within 2^-10 of a half-integer the quotient is recomputed in float64
            float q = __builtin_fmaf(x[m][c], dk.y, kMagic);
            const float lev = q - kMagic;
            const float fr = __builtin_fmaf(x[m][c], dk.y, -lev);
            if (__builtin_expect(fabsf(fabsf(fr) - 0.5f) <= 0x1.0p-10f, 0) && dk.x != 0.f)
                q = float(rint(double(x[m][c]) / double(dk.x))) + kMagic;
            q = __builtin_amdgcn_fmed3f(q, lo, hi);
            const uint32_t code = __float_as_uint(q) - (kMagicBits - uint32_t(n));   // level + n
            fld |= uint64_t(code) << (c * bw);
        }
        }
        const int off = sm.newoff[row] + cg * bw;
        const int wi = off >> 2, sh = (off & 3) * 8;
        const uint64_t lo64 = fld << sh;
        atomicOr(&sm.reg[wi], uint32_t(lo64));
        atomicOr(&sm.reg[wi + 1], uint32_t(lo64 >> 32));
        if (sh) {
            const uint32_t top = uint32_t(fld >> (64 - sh));
            if (top) atomicOr(&sm.reg[wi + 2], top);
        }
        if (cg == 0) {
            sm.newfit[row] = best;
            sm.newdelta[row] = dbits;
        }
    }
    __syncthreads();
    uint8_t* lb = reinterpret_cast<uint8_t*>(sm.reg);
    for (int row = tid; row < DK; row += NT) {
        reinterpret_cast<uint16_t*>(lb + code_bytes)[row] = sm.newdelta[row];
        lb[code_bytes + 2 * DK + row] = uint8_t((sm.newwidth[row] - 1) | (sm.newfit[row] << 4));
    }
    __syncthreads();
    for (int i = tid; i * 16 < total; i += NT)
        reinterpret_cast<uint4*>(region)[i] = reinterpret_cast<const uint4*>(sm.reg)[i];
}

// ---------------------------------------------------------------------------------
// Widths of one sequence's layer under the layer-wise budget ([LBRS] "State bit
// allocation": a layer-wise mean budget; "Range normalization": costs normalised per
// head, computed by the kCost pass): the geometric mean, the rounding, the clip and the
// one-bit adjustments of the per-head rule taken over all H*dk rows of the sequence,
// ties to the lower (head, row); when every head of the layer is zero every row keeps
// bbar. One workgroup per sequence; thread t owns the contiguous rows t*rpt ..
// t*rpt + rpt - 1, so that a row's rank among tied rows follows the thread order.
constexpr int LNT = 512, LMAX = 4096, LW = LNT / 64;   // up to 4096 rows

struct LayerSmem {
    double v0[LMAX];          // first candidate value of each row
    int8_t lim[LMAX];         // its number of candidates (one-bit steps)
    uint8_t bw[LMAX];         // widths
    double partd[2][LW];
    int parti[2][LW];
    uint32_t low_word;
};

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// block sums, summed over the wavefronts in a fixed order; `ph` alternates between
// the two slots so that one barrier per sum suffices
__device__ __forceinline__ double block_sum_f64(double v, LayerSmem& sm, int& ph) {
    v = wave_sum_f64<1>(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sm.partd[ph][wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < LW; ++w) t += sm.partd[ph][w];
    ph ^= 1;
    return t;
}
__device__ __forceinline__ int block_sum_i32(int v, LayerSmem& sm, int& ph) {
    v = wave_sum_i32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sm.parti[ph][wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < LW; ++w) t += sm.parti[ph][w];
    ph ^= 1;
    return t;
}

__global__ void __launch_bounds__(LNT) layer_widths_kernel(const AllocArgs A) {
    __shared__ LayerSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = A.rows_per_seq;
    const int rpt = (n + LNT - 1) / LNT;
    const int row0 = min(tid * rpt, n), row1 = min(row0 + rpt, n);
    const size_t base = (size_t)blockIdx.x * n;
    int ph = 0;
    int nz = 0;
    for (int r = row0; r < row1; ++r) {
        const double c = A.ws_c[base + r];
        sm.v0[r] = c;
        sm.bw[r] = uint8_t(A.bbar);
        nz += c != 0.0;
    }
    if (block_sum_i32(nz, sm, ph) > 0) {
        double lsum = 0.0;
        for (int r = row0; r < row1; ++r) {
            sm.v0[r] = fmax(sm.v0[r], 1e-300);
            lsum += log(sm.v0[r]);
        }
        const double gm = exp(block_sum_f64(lsum, sm, ph) / double(n));
        int tot = 0;
        for (int r = row0; r < row1; ++r) {
            const double bs = double(A.bbar) + 0.5 * log2(sm.v0[r] / gm);
            const int b = int(fmin(fmax(rint(bs), double(A.bmin)), double(A.bmax)));
            sm.bw[r] = uint8_t(b);
            tot += b;
        }
        const int target = A.bbar * n;
        tot = block_sum_i32(tot, sm, ph);
        const bool grow = tot < target;
        const int moves = grow ? target - tot : tot - target;
        if (moves > 0) {
            // candidates (row, step): the per-head rule's keys (gain bits, or the
            // complement of the loss bits), the `moves` largest taken; a row's
            // successive values scale exactly by `scale`
            const double scale = grow ? 0.25 : 4.0;
            for (int r = row0; r < row1; ++r) {
                const int b = sm.bw[r];
                const double c = sm.v0[r];
                sm.lim[r] = int8_t(grow ? A.bmax - b : b - A.bmin);
                sm.v0[r] = grow ? (0.75 * c) * exp2(-2.0 * b) : (3.0 * c) * exp2(-2.0 * b);
            }
            auto for_keys = [&](int r, auto f) {
                double v = sm.v0[r];
                const int lim = sm.lim[r];
                for (int st = 0; st < lim; ++st) {
                    const uint64_t bits = uint64_t(__double_as_longlong(v));
                    f(grow ? bits : ~bits);
                    v *= scale;
                }
            };
            auto count_if = [&](auto pred) {
                int cnt = 0;
                for (int r = row0; r < row1; ++r) for_keys(r, [&](uint64_t k) { cnt += pred(k); });
                return block_sum_i32(cnt, sm, ph);
            };
            uint32_t Hw = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = Hw | (1u << bit);
                if (count_if([&](uint64_t k) { return int(uint32_t(k >> 32) >= cand); }) >= moves) Hw = cand;
            }
            const uint64_t hiT = (uint64_t(Hw) << 32) | 0xFFFFFFFFull;
            const int need = moves - count_if([&](uint64_t k) { return int(k > hiT); });
            const int neq = count_if([&](uint64_t k) { return int(uint32_t(k >> 32) == Hw); });
            uint32_t Lw = 0;
            if (neq > 1) {
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t cand = Lw | (1u << bit);
                    if (count_if([&](uint64_t k) { return int(uint32_t(k >> 32) == Hw && uint32_t(k) >= cand); }) >= need)
                        Lw = cand;
                }
            } else {
                // the one key with that high word: its low word
                for (int r = row0; r < row1; ++r)
                    for_keys(r, [&](uint64_t k) {
                        if (uint32_t(k >> 32) == Hw) sm.low_word = uint32_t(k);
                    });
                __syncthreads();
                Lw = sm.low_word;
            }
            const uint64_t T = (uint64_t(Hw) << 32) | Lw;
            const int rem = moves - count_if([&](uint64_t k) { return int(k > T); });
            // this thread's tied rows (a row has at most one candidate equal to T: its
            // successive values differ by a factor of 4) and their rank in row order
            int ties = 0;
            for (int r = row0; r < row1; ++r) {
                bool t = false;
                for_keys(r, [&](uint64_t k) { t |= k == T; });
                ties += t;
            }
            int incl = ties;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            if (lane == 63) sm.parti[ph][wave] = incl;
            __syncthreads();
            int before = incl - ties;
            for (int w = 0; w < wave; ++w) before += sm.parti[ph][w];
            for (int r = row0; r < row1; ++r) {
                int a = 0;
                bool t = false;
                for_keys(r, [&](uint64_t k) {
                    a += k > T;
                    t |= k == T;
                });
                if (t) {
                    if (before < rem) ++a;
                    ++before;
                }
                sm.bw[r] = uint8_t(int(sm.bw[r]) + (grow ? a : -a));
            }
        }
    }
    for (int r = row0; r < row1; ++r) A.ws_w[base + r] = sm.bw[r];
}

// ---------------------------------------------------------------------------------
// Per-head allocation unit (HEADALLOC; [LBRS] "Allocation units": per-head decay and
// normalisation give each head one width and a scale per block of 32 key channels,
// R~ = 1, so decay alone sets the widths). The head's cost is the sum of its rows'
// persistence factors (under one width its proxy cost is sum_i Gamma_i 2^{-2b});
// the widths over the heads of a sequence come from layer_widths_kernel.
__global__ void __launch_bounds__(64) head_cost_kernel(const AllocArgs A) {
    const int head = blockIdx.x, lane = threadIdx.x;
    const size_t base = (size_t)head * DK;
    double g = 0.0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int row = 2 * lane + k;
        double s, q;
        bool flat = false;
        if (A.s) {
            s = A.s[base + row];
            q = A.r ? double(A.r[base + row]) : double(A.r_default);
        } else {
            const float* e = A.est + (size_t)head * est_stride(DK);
            const double W = e[2 * DK];
            flat = !(W > 0.0);
            s = -0.5 * log1p(-double(e[row]) / W);
            q = 0.5 * double(e[DK + row]) / W;
        }
        g += flat ? 1.0 : persistence(A.factor, A.cadence, s, q);
    }
    g = wave_sum_f64<1>(g);
    if (lane == 0) A.ws_c[head] = fmin(g, 1e300);
}

constexpr int HNG = DK / 32;                   // scale groups (32 rows) per column

struct HeadPackSmem {
    uint32_t old_codes[DK * DV / 4 + 4];
    uint32_t new_codes[DK * DV / 4 + 4];
    uint16_t scale[HNG * DV];
    uint8_t fit[HNG * DV];
    int old_width;
};

// Repack one head at the width the sequence pass chose: for each group (32 rows of one
// column, one thread) the clipping fit over f_k = 1/4 + k/20 at the new width (smallest
// squared error, ties to the larger f), Delta = f16(f R / n), the nearest levels.
__global__ void __launch_bounds__(NT) headalloc_pack_kernel(const AllocArgs A) {
    __shared__ HeadPackSmem sm;
    const int tid = threadIdx.x;
    const int head = blockIdx.x;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int cap = A.code_cap;
    if (tid == 0) sm.old_width = int(region[cap + 3 * HNG * DV]) + 1;
    for (int i = tid; i < HNG * DV / 8; i += NT)
        reinterpret_cast<uint4*>(sm.scale)[i] = reinterpret_cast<const uint4*>(region + cap)[i];
    for (int i = tid; i < DK * DV / 4 + 4; i += NT) sm.new_codes[i] = 0u;
    __syncthreads();
    const int bo = sm.old_width, bn = int(A.ws_w[head]);
    const int old_used = DK * DV * bo / 8, new_used = DK * DV * bn / 8;
    for (int i = tid; i * 16 < old_used; i += NT)
        reinterpret_cast<uint4*>(sm.old_codes)[i] = reinterpret_cast<const uint4*>(region)[i];
    if (tid < 4) sm.old_codes[old_used / 4 + tid] = 0u;
    __syncthreads();
    const int no = (1 << (bo - 1)) - 1, nn = (1 << (bn - 1)) - 1;
    for (int gi = tid; gi < HNG * DV; gi += NT) {
        const int g = gi / DV, col = gi - g * DV;
        const float dlo = f16_bits_to_f32(sm.scale[gi]);
        float x[32];
        float R = 0.f;
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) {
            const int bit = ((32 * g + rr) * DV + col) * bo;
            const uint64_t w = uint64_t(sm.old_codes[bit >> 5]) | (uint64_t(sm.old_codes[(bit >> 5) + 1]) << 32);
            const int field = int((w >> (bit & 31)) & ((1u << bo) - 1));
            x[rr] = float(field - no) * dlo;                 // exact: |level| <= 127 times a float16
            R = fmaxf(R, fabsf(x[rr]));
        }
        int best = 15;
        float be = 0.f;
        for (int k = 15; k >= 0; --k) {
            const float d = f16_bits_to_f32(f64_to_f16_bits(kFit.f[k] * double(R) / double(nn)));
            const float inv = d > 0.f ? 1.f / d : 0.f;
            float e = 0.f;
#pragma unroll
            for (int rr = 0; rr < 32; ++rr) {
                const float q = fminf(fmaxf(rintf(x[rr] * inv), -float(nn)), float(nn));
                const float r = __builtin_fmaf(-d, q, x[rr]);
                e = __builtin_fmaf(r, r, e);
            }
            if (k == 15 || e < be) {                          // ties keep the larger f
                be = e;
                best = k;
            }
        }
        const uint16_t dbits = f64_to_f16_bits(kFit.f[best] * double(R) / double(nn));
        const double d = double(f16_bits_to_f32(dbits));
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) {
            const int lev = d > 0.0 ? int(fmin(fmax(rint(double(x[rr]) / d), -double(nn)), double(nn))) : 0;
            const uint32_t field = uint32_t(lev + nn);
            const int bit = ((32 * g + rr) * DV + col) * bn;
            const int sh = bit & 31;
            atomicOr(&sm.new_codes[bit >> 5], field << sh);
            if (sh + bn > 32) atomicOr(&sm.new_codes[(bit >> 5) + 1], field >> (32 - sh));
        }
        sm.scale[gi] = dbits;
        sm.fit[gi] = uint8_t(best);
    }
    __syncthreads();
    // codes up to the longer of the old and the new length (the rest stays zero), then
    // the scales, the fit indices and the width
    const int span = old_used > new_used ? old_used : new_used;
    for (int i = tid; i * 16 < span; i += NT)
        reinterpret_cast<uint4*>(region)[i] = reinterpret_cast<const uint4*>(sm.new_codes)[i];
    for (int i = tid; i < HNG * DV / 8; i += NT)
        reinterpret_cast<uint4*>(region + cap)[i] = reinterpret_cast<const uint4*>(sm.scale)[i];
    for (int i = tid; i < HNG * DV / 16; i += NT)
        reinterpret_cast<uint4*>(region + cap + 2 * HNG * DV)[i] = reinterpret_cast<const uint4*>(sm.fit)[i];
    if (tid == 0) region[cap + 3 * HNG * DV] = uint8_t(bn - 1);
}

}  // namespace

hipError_t launch_allocate_bits(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    if (d.bmin == 1) hipLaunchKernelGGL((allocate_kernel<kHead, true, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((allocate_kernel<kHead, false, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int MODE, bool SR>
void launch_alloc_ob(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    if (d.bmin == 1) hipLaunchKernelGGL((allocate_kernel<MODE, true, SR>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((allocate_kernel<MODE, false, SR>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
}

template <bool SR>
hipError_t step_allocate(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    if (d.budget != WB_BUDGET_LAYER) {
        launch_alloc_ob<kStep, SR>(d, a, stream);
        return hipGetLastError();
    }
    // layer budget: step and costs, the widths of each sequence, then the step again
    // with the fit and the rounding at those widths
    launch_alloc_ob<kStepCost, SR>(d, a, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layer_widths_kernel, dim3(d.B), dim3(LNT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_alloc_ob<kStepPack, SR>(d, a, stream);
    return hipGetLastError();
}

hipError_t launch_step_allocate(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    return d.mode == WB_SR ? step_allocate<true>(d, a, stream) : step_allocate<false>(d, a, stream);
}

hipError_t launch_allocate_heads(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(head_cost_kernel, dim3(d.B * d.H), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layer_widths_kernel, dim3(d.B), dim3(LNT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(headalloc_pack_kernel, dim3(d.B * d.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_allocate_layer(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    if (d.bmin == 1) hipLaunchKernelGGL((allocate_kernel<kCost, true, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((allocate_kernel<kCost, false, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layer_widths_kernel, dim3(d.B), dim3(LNT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d.bmin == 1) hipLaunchKernelGGL((allocate_kernel<kPack, true, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((allocate_kernel<kPack, false, false>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wb
