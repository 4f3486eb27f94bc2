// Prefill with deferred write-back (chunked gated delta rule on MFMA).
//
// [LBRS] "Accumulated readout error": write-back happens once every C tokens (per
// prefill chunk, per token in decode, or deferred with C = 8); outputs are read from
// the unquantized state before each write-back. Between two write-backs the state
// evolves exactly, so each call is cut into segments of at most 8 tokens that end at
// every write-back point; a segment of L tokens starting from state S_0 is evaluated
// in closed form (a WY-style rewrite of L delta-rule steps):
//   g_t = sum_{tau<=t} s_tau (per key row), Gamma_t = e^{-g_t};
//   k^_t = Gamma_t k_t,  q^_t = Gamma_t q_t,  k-_t = k_t / Gamma_t;
//   w_t  = beta_t (v_t - S_0^T k^_t - sum_{tau<t} (k^_t . k-_tau) w_tau)   (forward solve)
//   o_t  = S_0^T q^_t + sum_{tau<=t} (q^_t . k-_tau) w_tau
//   S_L  = Gamma_L S_0 + sum_tau (Gamma_L k-_tau) w_tau^T.
// The dense contractions [k^; q^] S_0 (16 x 128 x 128) and the rank-8 update run on
// v_mfma_f32_16x16x4_f32 in float32 (inputs q, k, v are bfloat16); the triangular
// solve and the small dot products run on the vector ALUs.
//
// State placement: the 128 x 128 state lives in registers in the MFMA accumulator
// layout. Wave w owns columns 32w .. 32w+31 (2 column tiles of 16) and all 8 row tiles;
// lane l holds rows 16*rt + 4*(l/16) + r (r = 0..3) of columns 32w + 16*ct + l%16. The
// same registers serve as the B operand of the [k^; q^] S_0 contraction (K index =
// row), so no state data moves between waves. Hadamard rows stay rotated (Y = S H):
// the contraction over rotated rows is transformed back with one 128-point transform
// per output vector, and rotated rows are updated with H w.
//
// Write-back (every C tokens and after the last token) rounds the register state in
// place: float16 rows to nearest float16; Hadamard INT8 rows per block of 32 columns
// (= one wave's columns) with an asymmetric affine grid ([DAMP] "Quantization &
// calibration details"); uniform rows on the B-bit grid. The last write-back is also
// encoded into the stored region. Supported here: FP32, UNIFORM, HAD_INT8 and MIXED
// with affine blocks of 32 values, round-to-nearest.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256, SEG = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));   // MFMA accumulator fragment
constexpr float kInvSqrt128f = 0.08838834764831845f;

struct PfSmem {
    float khat[SEG][DK];      // rows 0..7 of the contraction operand
    float qhat[SEG][DK];      // rows 8..15 (must follow khat)
    float kbar[SEG][DK];      // k_tau / Gamma_tau
    float kbarL[SEG][DK];     // Gamma_L k_tau / Gamma_tau
    float gl[DK];             // Gamma_L per row
    float kqt[DK][20];        // [k^; q^] transposed (16 used): the MFMA A operand, read
                              // without bank conflicts (row stride 20 floats)
    float v[SEG][DV];
    float ks[2 * SEG][DV];    // [k^; q^] S_0 over the unrotated rows, then the whole contraction
    float ksq[2 * SEG][DV];   // the same over the rotated rows
    float w[SEG][DV];
    float hw[SEG][DV];
    float A[SEG][SEG], QK[SEG][SEG];
    float beta[SEG];
    int perm[DK];
    float wbuf[DK][DV + 4];   // the state in row-major order for the write-back (row stride
                              // padded to 132 floats: both transposes are conflict-free)
};

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Butterfly partner at lane ^ d for d = 1, 2, 4, 8 (DPP inside a row of 16 lanes),
// 16 and 32 (lane swaps of the odd and even rows or of the two halves: swapping a
// register with itself leaves the even rows' (low half's) values in the first result
// and the odd rows' (high half's) in the second, everywhere).
template <int D>
__device__ __forceinline__ float xor_partner(float v, int lane) {
    const int b = __float_as_int(v);
    if constexpr (D == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false));
    if constexpr (D == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false));
    if constexpr (D == 4) {
        // row_ror:n hands lane i the value of lane i - n (mod 16)
        const int up = __builtin_amdgcn_mov_dpp(b, 0x12C, 0xF, 0xF, false);     // row_ror:12 (i + 4)
        const int dn = __builtin_amdgcn_mov_dpp(b, 0x124, 0xF, 0xF, false);     // row_ror:4  (i - 4)
        return __int_as_float((lane & 4) ? dn : up);
    }
    if constexpr (D == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, false));   // row_ror:8
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    const auto r = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

template <int D>
__device__ __forceinline__ void butterfly(float& x, float& y, int lane) {
    const float sg = (lane & D) ? -1.f : 1.f;     // lane with bit D set: partner - self
    const float ox = xor_partner<D>(x, lane), oy = xor_partner<D>(y, lane);
    x = __builtin_fmaf(sg, x, ox);
    y = __builtin_fmaf(sg, y, oy);
}

// 128-point orthonormal transform of a vector held by one wavefront as v[lane], v[lane + 64]
__device__ __forceinline__ void wave_wht128(float& a0, float& a1, int lane) {
    float x = a0 + a1, y = a0 - a1;
    butterfly<1>(x, y, lane);
    butterfly<2>(x, y, lane);
    butterfly<4>(x, y, lane);
    butterfly<8>(x, y, lane);
    butterfly<16>(x, y, lane);
    butterfly<32>(x, y, lane);
    a0 = x * kInvSqrt128f;
    a1 = y * kInvSqrt128f;
}

template <int KIND>
struct PfLayout {
    static constexpr bool ROT = KIND == WB_HAD_INT8 || KIND == WB_MIXED;
    // row tile rt is rotated (Hadamard) for these layouts; MIXED keeps row tile 0
    // (physical rows 0..15, the float16 rows with k_hi = 16) unrotated
    __device__ static bool rotated(int rt) { return KIND == WB_HAD_INT8 || (KIND == WB_MIXED && rt > 0); }
};

// One segment's inputs as this thread reads them: thread t owns physical row t % 128
// for the tokens 4 (t / 128) .. +3 (k and q; the decays of all the segment's tokens),
// every thread owns 4 values of v, and threads 0..7 one beta each. Loaded a segment
// ahead into registers.
struct SegIn {
    uint16_t kk[SEG / 2], qq[SEG / 2];
    float sv[SEG];
    uint16_t vv[SEG * DV / NT];
    float beta;
};

__device__ __forceinline__ void load_segment(const PrefillArgs& P, int b, int h, int t, int L, int tid, int lr,
                                             SegIn& in) {
    const KArgs& A = P.base;
    const int H = A.H, T = P.T;
    const int half = tid / DK;
#pragma unroll
    for (int tt = 0; tt < SEG; ++tt) {
        in.sv[tt] = 0.f;
        if (tt < L) {
            const size_t base = ((size_t)b * T + t + tt) * H + h;
            in.sv[tt] = A.s_per_row ? P.s[base * DK + lr] : P.s[base];
        }
    }
#pragma unroll
    for (int t4 = 0; t4 < SEG / 2; ++t4) {
        const int tt = (SEG / 2) * half + t4;
        in.kk[t4] = 0;
        in.qq[t4] = 0;
        if (tt < L) {
            const size_t base = ((size_t)b * T + t + tt) * H + h;
            in.kk[t4] = P.k[base * DK + lr];
            in.qq[t4] = P.q[base * DK + lr];
        }
    }
#pragma unroll
    for (int n = 0; n < SEG * DV / NT; ++n) {
        const int i = tid + n * NT, tt = i / DV, j = i - tt * DV;
        in.vv[n] = tt < L ? P.v[(((size_t)b * T + t + tt) * H + h) * DV + j] : uint16_t(0);
    }
    in.beta = (tid < SEG && tid < L) ? P.beta[((size_t)b * T + t + tid) * H + h] : 0.f;
}

// length of the segment starting at t: up to SEG tokens, ending at the next
// write-back point or the last token
__device__ __forceinline__ int segment_length(int t, int T, int C) {
    const int to_wb = C - (t % C);
    int L = SEG < to_wb ? SEG : to_wb;
    return L > T - t ? T - t : L;
}

template <int KIND>
__global__ void __launch_bounds__(NT) prefill_kernel(const PrefillArgs P) {
    __shared__ PfSmem sm;
    using LY = PfLayout<KIND>;
    const KArgs& A = P.base;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int head = blockIdx.x;
    const int H = A.H;
    const int b = head / H, h = head - b * H;
    const int lc = lane & 15, lg = lane >> 4;          // column within tile, row group
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int k_hi = (KIND == WB_MIXED) ? A.k_hi : 0;
    const size_t code_base = (size_t)k_hi * DV * 2;
    const size_t meta_base = code_base + (size_t)(DK - k_hi) * DV;
    const int ub = A.bits;
    const float ustep = 1.f / float(1 << (ub - 1));

    for (int i = tid; i < DK; i += NT) sm.perm[i] = (KIND == WB_MIXED) ? int(A.perm[h * DK + i]) : i;

    // ---- load and dequantize the stored state into the accumulator layout ----------
    f32x4 S[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            float e[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * lg + r;
                const int col = 32 * wave + 16 * ct + lc;
                float x = 0.f;
                if (KIND == WB_FP32) {
                    x = reinterpret_cast<const float*>(region)[row * DV + col];
                } else if (KIND == WB_UNIFORM) {
                    const int bit = (row * DV + col) * ub;
                    const uint32_t byte = region[bit >> 3];
                    int kap = int((byte >> (bit & 7)) & ((1u << ub) - 1));
                    if (kap >= (1 << (ub - 1))) kap -= (1 << ub);
                    x = float(kap) * ustep;
                } else if (KIND == WB_MIXED && row < k_hi) {
                    x = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(region)[row * DV + col]);
                } else {
                    const int qrow = row - k_hi;
                    const uint32_t code = region[code_base + (size_t)qrow * DV + col];
                    const uint32_t sz = *reinterpret_cast<const uint32_t*>(
                        region + meta_base + ((size_t)qrow * (DV / 32) + col / 32) * 4);
                    x = f16_bits_to_f32(sz >> 16) + float(code) * f16_bits_to_f32(sz & 0xFFFFu);
                }
                e[r] = x;
            }
            S[rt][ct] = f32x4{e[0], e[1], e[2], e[3]};
        }
    __syncthreads();

    const int T = P.T;
    const int my_lr = sm.perm[tid & (DK - 1)];
    SegIn nxt;
    load_segment(P, b, h, 0, segment_length(0, T, P.C), tid, my_lr, nxt);
    int t = 0;
    while (t < T) {
        const int L = segment_length(t, T, P.C);
        const bool write_back = ((t + L) % P.C == 0) || (t + L == T);
        const SegIn cur = nxt;

        // ---- stage inputs (physical row order) and the decay products ---------------
#pragma unroll
        for (int n = 0; n < SEG * DV / NT; ++n) {
            const int i = tid + n * NT, tt = i / DV, j = i - tt * DV;
            sm.v[tt][j] = bf16f(cur.vv[n]);
        }
        if (tid < SEG) sm.beta[tid] = cur.beta;
        {
            // thread t: row t % 128, tokens 4 (t / 128) .. +3
            const int p = tid & (DK - 1), half = tid / DK;
            float g[SEG];
            float acc = 0.f;
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                acc += cur.sv[tt];
                g[tt] = acc;
            }
            const float gL = g[L - 1];
            const float decL = expf(-gL);
#pragma unroll
            for (int t4 = 0; t4 < SEG / 2; ++t4) {
                const int tt = (SEG / 2) * half + t4;
                const float gt = half ? g[SEG / 2 + t4] : g[t4];
                const float kk = bf16f(cur.kk[t4]), qq = bf16f(cur.qq[t4]);
                const float dec = __expf(-gt);       // hardware exp2 of the scaled argument
                const float inc = __builtin_amdgcn_rcpf(dec);      // e^{g}, within an ulp or two
                sm.khat[tt][p] = kk * dec;
                sm.qhat[tt][p] = qq * dec;
                sm.kqt[p][tt] = kk * dec;
                sm.kqt[p][SEG + tt] = qq * dec;
                sm.kbar[tt][p] = kk * inc;
                sm.kbarL[tt][p] = kk * (inc * decL);
            }
            if (half == 0) sm.gl[p] = decL;
        }
        __syncthreads();
        // small Gram matrices: A[t][tau] = k^_t . k-_tau (tau < t), QK[t][tau] (tau <= t);
        // four lanes (a DPP quad) per entry, 32 rows each
        {
            const int pair = tid >> 2, part = tid & 3;
            const int tt = pair / SEG, ta = pair - tt * SEG;
            float a = 0.f, q = 0.f;
            if (ta <= tt && tt < L) {
                const float4* kh = reinterpret_cast<const float4*>(&sm.khat[tt][32 * part]);
                const float4* qh = reinterpret_cast<const float4*>(&sm.qhat[tt][32 * part]);
                const float4* kb = reinterpret_cast<const float4*>(&sm.kbar[ta][32 * part]);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 x = kh[i], y = qh[i], z = kb[i];
                    a = __builtin_fmaf(x.x, z.x, a); a = __builtin_fmaf(x.y, z.y, a);
                    a = __builtin_fmaf(x.z, z.z, a); a = __builtin_fmaf(x.w, z.w, a);
                    q = __builtin_fmaf(y.x, z.x, q); q = __builtin_fmaf(y.y, z.y, q);
                    q = __builtin_fmaf(y.z, z.z, q); q = __builtin_fmaf(y.w, z.w, q);
                }
            }
            a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false));
            q += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(q), 0xB1, 0xF, 0xF, false));
            a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false));
            q += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(q), 0x4E, 0xF, 0xF, false));
            if (part == 0) {
                sm.A[tt][ta] = (ta < tt) ? a : 0.f;
                sm.QK[tt][ta] = (ta <= tt) ? q : 0.f;
            }
        }

        // ---- [k^; q^] S_0 on MFMA (16 x 32 per wave), rotated rows kept apart --------
        f32x4 accP[2], accQ[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            accP[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            accQ[ct] = accP[ct];
        }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = sm.kqt[16 * rt + 4 * lg + r][lc];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const float bv = (r == 0) ? S[rt][ct].x : (r == 1) ? S[rt][ct].y : (r == 2) ? S[rt][ct].z : S[rt][ct].w;
                    if (LY::rotated(rt))
                        accQ[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, accQ[ct], 0, 0, 0);
                    else
                        accP[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, accP[ct], 0, 0, 0);
                }
            }
        }
        // accumulator element (M = 4*lg + r, column 32w + 16ct + lc)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = 32 * wave + 16 * ct + lc;
            sm.ks[4 * lg + 0][col] = accP[ct].x;
            sm.ks[4 * lg + 1][col] = accP[ct].y;
            sm.ks[4 * lg + 2][col] = accP[ct].z;
            sm.ks[4 * lg + 3][col] = accP[ct].w;
            if (LY::ROT) {
                sm.ksq[4 * lg + 0][col] = accQ[ct].x;
                sm.ksq[4 * lg + 1][col] = accQ[ct].y;
                sm.ksq[4 * lg + 2][col] = accQ[ct].z;
                sm.ksq[4 * lg + 3][col] = accQ[ct].w;
            }
        }
        __syncthreads();
        if (LY::ROT) {
            // wave w transforms vectors 4w .. 4w+3 back from the rotated domain and adds
            // the unrotated part
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int m = 4 * wave + vv;
                float a0 = sm.ksq[m][lane], a1 = sm.ksq[m][lane + 64];
                wave_wht128(a0, a1, lane);
                sm.ks[m][lane] += a0;
                sm.ks[m][lane + 64] += a1;
            }
            __syncthreads();
        }

        // ---- per column: forward solve for w (threads 0..127) ------------------------
        if (tid < DV) {
            const int j = tid;
            float wv[SEG];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                float u = sm.v[tt][j] - sm.ks[tt][j];
#pragma unroll
                for (int ta = 0; ta < tt; ++ta) u = __builtin_fmaf(-sm.A[tt][ta], wv[ta], u);
                wv[tt] = sm.beta[tt] * u;
                sm.w[tt][j] = wv[tt];
            }
        }
        // inputs of the next segment (requested before this segment's output stores)
        if (t + L < T) load_segment(P, b, h, t + L, segment_length(t + L, T, P.C), tid, my_lr, nxt);
        __syncthreads();
        // ---- outputs o (threads 128..255) beside H w (threads 0..127) ------------------
        if (tid >= NT - DV) {
            const int j = tid - (NT - DV);
            float wv[SEG];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) wv[tt] = sm.w[tt][j];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                if (tt < L) {
                    float o = sm.ks[SEG + tt][j];
#pragma unroll
                    for (int ta = 0; ta <= tt; ++ta) o = __builtin_fmaf(sm.QK[tt][ta], wv[ta], o);
                    P.o[(((size_t)b * T + t + tt) * H + h) * DV + j] = o;
                }
            }
        } else if (LY::ROT) {
            // H w for the rotated rows: four vectors per wave
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int m = 4 * wave + vv;
                float a0 = sm.w[m][lane], a1 = sm.w[m][lane + 64];
                wave_wht128(a0, a1, lane);
                sm.hw[m][lane] = a0;
                sm.hw[m][lane + 64] = a1;
            }
        }
        if (LY::ROT) __syncthreads();

        // ---- S_L = Gamma_L S_0 + sum_tau (Gamma_L k-_tau) w_tau^T  (MFMA, K = 8) ------
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const float g0 = sm.gl[16 * rt + 4 * lg + 0], g1 = sm.gl[16 * rt + 4 * lg + 1];
            const float g2 = sm.gl[16 * rt + 4 * lg + 2], g3 = sm.gl[16 * rt + 4 * lg + 3];
            const float* wsrc = LY::rotated(rt) ? &sm.hw[0][0] : &sm.w[0][0];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4 c = S[rt][ct];
                c.x *= g0;
                c.y *= g1;
                c.z *= g2;
                c.w *= g3;
                const int col = 32 * wave + 16 * ct + lc;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int tok = 4 * kk + lg;
                    const float a = sm.kbarL[tok][16 * rt + lc];
                    const float bv = wsrc[tok * DV + col];
                    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, c, 0, 0, 0);
                }
                S[rt][ct] = c;
            }
        }

        // ---- write-back ---------------------------------------------------------------
        // The state goes through LDS in row-major order: each thread then rounds two
        // whole 32-value row blocks (one INT8 block each: extrema, float16 metadata and
        // levels without cross-lane steps), and the call's last write-back stores its
        // codes contiguously.
        if (write_back && KIND != WB_FP32) {
            const bool last = (t + L == T);
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int col = 32 * wave + 16 * ct + lc;
                    const f32x4 v = S[rt][ct];
                    sm.wbuf[16 * rt + 4 * lg + 0][col] = v.x;
                    sm.wbuf[16 * rt + 4 * lg + 1][col] = v.y;
                    sm.wbuf[16 * rt + 4 * lg + 2][col] = v.z;
                    sm.wbuf[16 * rt + 4 * lg + 3][col] = v.w;
                }
            __syncthreads();
#pragma unroll
            for (int unit = 0; unit < 2; ++unit) {
                const int u = tid + NT * unit;
                const int row = u >> 2, cb = u & 3;          // row block: columns 32 cb .. +31
                float4* rp = reinterpret_cast<float4*>(&sm.wbuf[row][32 * cb]);
                float x[32];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 f = rp[i];
                    x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
                }
                if (KIND == WB_UNIFORM) {
                    const float lo = -float(1 << (ub - 1)), hi = float((1 << (ub - 1)) - 1);
                    const float inv = float(1 << (ub - 1));
                    float kv[32];
#pragma unroll
                    for (int c = 0; c < 32; ++c) {
                        kv[c] = fminf(fmaxf(rintf(x[c] * inv), lo), hi);
                        x[c] = kv[c] * ustep;
                    }
                    if (last) {
                        // codes are packed only where they are stored
                        uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // 32 fields of ub <= 8 bits
#pragma unroll
                        for (int c = 0; c < 32; ++c) {
                            const int bit = c * ub;
                            wd[bit >> 5] |= (uint32_t(int(kv[c])) & ((1u << ub) - 1)) << (bit & 31);
                        }
                        // element (row, col) at bit ub (row DV + col): this block is 4 ub
                        // contiguous bytes, 4-byte aligned
                        uint32_t* dst = reinterpret_cast<uint32_t*>(region + ((row * DV + 32 * cb) * ub) / 8);
                        for (int i = 0; i < ub; ++i) dst[i] = wd[i];
                    }
                } else if (KIND == WB_MIXED && row < k_hi) {
                    uint32_t hw2[16];
#pragma unroll
                    for (int c = 0; c < 32; c += 2) {
                        const uint16_t h0 = f32_to_f16_bits(x[c]), h1 = f32_to_f16_bits(x[c + 1]);
                        x[c] = f16_bits_to_f32(h0);
                        x[c + 1] = f16_bits_to_f32(h1);
                        hw2[c >> 1] = uint32_t(h0) | (uint32_t(h1) << 16);
                    }
                    if (last) {
                        uint4* dst = reinterpret_cast<uint4*>(region + (row * DV + 32 * cb) * 2);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dst[i] = make_uint4(hw2[4 * i], hw2[4 * i + 1], hw2[4 * i + 2], hw2[4 * i + 3]);
                    }
                } else {
                    // affine INT8 block of 32 values
                    float mn = x[0], mx = x[0];
#pragma unroll
                    for (int c = 1; c < 32; ++c) {
                        mn = fminf(mn, x[c]);
                        mx = fmaxf(mx, x[c]);
                    }
                    const uint32_t sb = f16_bits_of_product(fmaxf(mx - mn, 0.f), 1.f / 255.f);
                    const uint16_t zb = f32_to_f16_bits(mn);
                    const float sc = f16_bits_to_f32(sb), ze = f16_bits_to_f32(zb);
                    // levels in magic-number form (1.5 * 2^23 + level); level 0 if the
                    // block is constant
                    constexpr float M = 12582912.0f;
                    float yv[32];
                    if (sc > 0.f) {
                        // reciprocal refined by one Newton step; rounding by adding 1.5 * 2^23
                        // (ties to even), clamp by med3
                        float inv = __builtin_amdgcn_rcpf(sc);
                        inv = __builtin_fmaf(__builtin_fmaf(-sc, inv, 1.f), inv, inv);
#pragma unroll
                        for (int c = 0; c < 32; ++c) {
                            yv[c] = __builtin_amdgcn_fmed3f(__builtin_fmaf(x[c] - ze, inv, M), M, M + 255.f);
                            x[c] = __builtin_fmaf(yv[c] - M, sc, ze);
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < 32; ++c) {
                            yv[c] = M;
                            x[c] = ze;
                        }
                    }
                    if (last) {
                        // codes are packed only where they are stored
                        uint32_t cw4[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                        for (int c = 0; c < 32; ++c) cw4[c >> 2] |= (__float_as_uint(yv[c]) & 0xFFu) << (8 * (c & 3));
                        const int qrow = row - k_hi;
                        uint4* dst = reinterpret_cast<uint4*>(region + code_base + (size_t)qrow * DV + 32 * cb);
                        dst[0] = make_uint4(cw4[0], cw4[1], cw4[2], cw4[3]);
                        dst[1] = make_uint4(cw4[4], cw4[5], cw4[6], cw4[7]);
                        *reinterpret_cast<uint32_t*>(region + meta_base + ((size_t)qrow * (DV / 32) + cb) * 4) =
                            uint32_t(sb) | (uint32_t(zb) << 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) rp[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
            }
            __syncthreads();
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int col = 32 * wave + 16 * ct + lc;
                    S[rt][ct] = f32x4{sm.wbuf[16 * rt + 4 * lg + 0][col], sm.wbuf[16 * rt + 4 * lg + 1][col],
                                      sm.wbuf[16 * rt + 4 * lg + 2][col], sm.wbuf[16 * rt + 4 * lg + 3][col]};
                }
        }
        if (KIND == WB_FP32 && t + L == T) {
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int col = 32 * wave + 16 * ct + lc;
                    float* dst = reinterpret_cast<float*>(region);
                    dst[(16 * rt + 4 * lg + 0) * DV + col] = S[rt][ct].x;
                    dst[(16 * rt + 4 * lg + 1) * DV + col] = S[rt][ct].y;
                    dst[(16 * rt + 4 * lg + 2) * DV + col] = S[rt][ct].z;
                    dst[(16 * rt + 4 * lg + 3) * DV + col] = S[rt][ct].w;
                }
        }
        __syncthreads();
        t += L;
    }
}

}  // namespace

hipError_t launch_prefill(const wb_layout_desc& d, const PrefillArgs& a, hipStream_t stream) {
    if (d.dk != 128 || d.dv != 128 || d.mode != WB_RTN || d.int_bits == 4) return hipErrorNotSupported;
    const dim3 grid(d.B * d.H), block(NT);
    switch (d.kind) {
        case WB_FP32: hipLaunchKernelGGL(prefill_kernel<WB_FP32>, grid, block, 0, stream, a); break;
        case WB_UNIFORM: hipLaunchKernelGGL(prefill_kernel<WB_UNIFORM>, grid, block, 0, stream, a); break;
        case WB_HAD_INT8:
            if (d.block != 32) return hipErrorNotSupported;
            hipLaunchKernelGGL(prefill_kernel<WB_HAD_INT8>, grid, block, 0, stream, a);
            break;
        case WB_MIXED:
            if (d.block != 32 || d.k_hi != 16) return hipErrorNotSupported;
            hipLaunchKernelGGL(prefill_kernel<WB_MIXED>, grid, block, 0, stream, a);
            break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace wb
