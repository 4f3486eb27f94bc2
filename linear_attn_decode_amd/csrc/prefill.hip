// Prefill with deferred write-back (chunked gated delta rule on MFMA).
//
// [LBRS] "Accumulated readout error": write-back happens once every C tokens (per
// prefill chunk, per token in decode, or deferred with C = 8); outputs are read from
// the unquantized state before each write-back; [LBRS] "Protocol": each write-back is
// quantized and dequantized before the state is used again. Between two write-backs the
// state evolves exactly, so each call is cut into segments that end at every
// write-back point (and at most min(chunk, 8) tokens long); a segment of L tokens
// starting from state S_0 is evaluated in closed form (a WY-style rewrite of L
// delta-rule steps):
//   g_t = sum_{tau<=t} s_tau (per key row), Gamma_t = e^{-g_t};
//   k^_t = Gamma_t k_t,  q^_t = Gamma_t q_t,  k-_t = k_t / Gamma_t;
//   w_t  = beta_t (v_t - S_0^T k^_t - sum_{tau<t} (k^_t . k-_tau) w_tau)   (forward solve)
//   o_t  = S_0^T q^_t + sum_{tau<=t} (q^_t . k-_tau) w_tau
//   S_L  = Gamma_L S_0 + sum_tau (Gamma_L k-_tau) w_tau^T.
// The dense contractions [k^; q^] S_0 (16 x 128 x 128) and the rank-8 update run on
// the matrix cores; the Gram matrices, the triangular solve and the transforms on the
// vector ALUs.
//
// Precision: the state path runs in float64 (v_mfma_f64_16x16x4_f64 for both
// contractions, float64 decay factors, Gram matrices, solve and transforms). A
// write-back decides a stored code to within 1e-5 of a step; on 8-bit grids and float16
// rows that is below one float32 ulp of the value, so a float32 state path flips codes
// the float64 recurrence does not, and the trajectories of a long call diverge. Outputs
// are stored as float32.
//
// State placement: the 128 x 128 state lives in registers in the float64 MFMA
// accumulator layout, over 8 wavefronts (2 per SIMD, so that one hides the other's
// latency). Wave w owns columns 16w .. 16w+15 (one column tile) and all 8 row tiles;
// register r of lane l holds row 16*rt + l/16 + 4*r (r = 0..3) of column 16w + l%16
// (the float64 16 x 16 result interleaves its rows over the four lane groups, unlike
// the float32 one, which gives each lane group 4 consecutive rows). The
// same registers serve as the B operand of the [k^; q^] S_0 contraction (K index =
// row), so no state data moves between waves. Hadamard rows stay rotated (Y = S H):
// the contraction over rotated rows is transformed back with one 128-point transform
// per output vector, and rotated rows are updated with H w.
//
// Write-back (every C tokens and after the last token) rounds the state in place,
// through LDS in two halves of 64 rows (two threads per 32-value row block): float16
// rows to the nearest float16; Hadamard INT8 rows per block of 32 columns on an
// asymmetric affine grid ([DAMP] "Quantization & calibration details");
// uniform rows on the B-bit grid. The last write-back is also encoded into the stored
// region. Supported here: FP32, UNIFORM, HAD_INT8 and MIXED with affine blocks of 32
// values, round-to-nearest.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NW = 8, NT = 64 * NW, SEG = 8;
typedef double f64x4 __attribute__((ext_vector_type(4)));   // MFMA accumulator fragment
constexpr double kInvSqrt128 = 0.088388347648318440550;     // 1 / sqrt(128)

// LDS strides (in doubles) chosen against bank conflicts of 64-bit accesses, taken per
// half wavefront (32 lanes, 32 double-wide bank pairs):
//   * PS:  rows of k^, q^, k- as 8 parts of 16 rows padded to 17 (the Gram threads read
//          4 tokens x 8 parts per half wavefront: slots 8 token + 17 part, all distinct);
//   * VS:  vectors over the value axis read by two lane groups at once (rows 16 apart
//          in slots: 128 + 16);
//   * KQS: the transposed [k^; q^] (odd, so a row's 16 entries and the next row's
//          do not collide);
//   * WBS: the write-back copy, row blocks of 32 padded to 33 (132 = 4 mod 32): the
//          block threads (4 rows x 4 blocks x 2 halves per half wavefront) read
//          distinct slots.
constexpr int PS = 8 * 17, VS = DV + 16, KQS = 17, WBS = 4 * 33;
__device__ __forceinline__ int pidx(int row) { return (row >> 4) * 17 + (row & 15); }    // row in a PS row
__device__ __forceinline__ int widx(int col) { return (col >> 5) * 33 + (col & 31); }    // column in a WBS row

// per-segment staging (dead while the write-back uses the same storage)
struct PfStage {
    double khat[SEG][PS];
    double qhat[SEG][PS];
    double kbar[SEG][PS];      // k_tau / Gamma_tau
    double kbarL[SEG][VS];     // Gamma_L k_tau / Gamma_tau
    double kqt[DK][KQS];       // [k^; q^] transposed (16 used): the MFMA A operand
    double ks[2 * SEG][VS];    // [k^; q^] S_0 over the unrotated rows, then the whole contraction
    double ksq[2 * SEG][VS];   // the same over the rotated rows
};
struct PfSmem {
    union {
        PfStage st;
        double wbuf[DK / 2][WBS];   // half of the state, row-major, for the write-back
    } u;
    float v[SEG][DV];
    double w[SEG][VS];
    double hw[SEG][VS];
    double gl[DK];             // Gamma_L per row
    double A[SEG][SEG], QK[SEG][SEG];
    double beta[SEG];
    int perm[DK];
};

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ double f16d(uint32_t bits) { return double(f16_bits_to_f32(bits)); }

// DPP move of a float64 inside rows of 16 lanes (both halves)
template <int CTRL>
__device__ __forceinline__ double mov_dpp_f64(double v) {
    const uint64_t b = uint64_t(__double_as_longlong(v));
    const uint32_t lo = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

// Butterfly partner at lane ^ d for d = 1, 2, 4, 8 (DPP inside a row of 16 lanes),
// 16 and 32 (lane swaps of the odd and even rows or of the two halves: swapping a
// register with itself leaves the even rows' (low half's) values in the first result
// and the odd rows' (high half's) in the second, everywhere).
template <int D>
__device__ __forceinline__ double xor_partner(double v, int lane) {
    if constexpr (D == 1) return mov_dpp_f64<0xB1>(v);
    if constexpr (D == 2) return mov_dpp_f64<0x4E>(v);
    if constexpr (D == 4) {
        // row_ror:n hands lane i the value of lane i - n (mod 16)
        const double up = mov_dpp_f64<0x12C>(v);     // row_ror:12 (i + 4)
        const double dn = mov_dpp_f64<0x124>(v);     // row_ror:4  (i - 4)
        return (lane & 4) ? dn : up;
    }
    if constexpr (D == 8) return mov_dpp_f64<0x128>(v);   // row_ror:8
    const uint64_t b = uint64_t(__double_as_longlong(v));
    if constexpr (D == 16) {
        const auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
        const bool up = lane & 16;
        return __longlong_as_double((long long)((uint64_t(up ? hi[0] : hi[1]) << 32) | (up ? lo[0] : lo[1])));
    }
    const auto lo = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
    const bool up = lane & 32;
    return __longlong_as_double((long long)((uint64_t(up ? hi[0] : hi[1]) << 32) | (up ? lo[0] : lo[1])));
}

template <int D>
__device__ __forceinline__ void butterfly(double& x, double& y, int lane) {
    const double ox = xor_partner<D>(x, lane), oy = xor_partner<D>(y, lane);
    // lane with bit D set: partner - self
    if (lane & D) {
        x = ox - x;
        y = oy - y;
    } else {
        x = x + ox;
        y = y + oy;
    }
}

// 128-point orthonormal transform of a vector held by one wavefront as v[lane], v[lane + 64]
__device__ __forceinline__ void wave_wht128(double& a0, double& a1, int lane) {
    double x = a0 + a1, y = a0 - a1;
    butterfly<1>(x, y, lane);
    butterfly<2>(x, y, lane);
    butterfly<4>(x, y, lane);
    butterfly<8>(x, y, lane);
    butterfly<16>(x, y, lane);
    butterfly<32>(x, y, lane);
    a0 = x * kInvSqrt128;
    a1 = y * kInvSqrt128;
}

template <int KIND>
struct PfLayout {
    static constexpr bool ROT = KIND == WB_HAD_INT8 || KIND == WB_MIXED;
    // row tile rt is rotated (Hadamard) for these layouts; MIXED keeps row tile 0
    // (physical rows 0..15, the float16 rows with k_hi = 16) unrotated
    __device__ static bool rotated(int rt) { return KIND == WB_HAD_INT8 || (KIND == WB_MIXED && rt > 0); }
};

// One segment's inputs as this thread reads them: thread t owns physical row t % 128
// for the tokens 2 (t / 128), +1 (k and q; the decays of all the segment's tokens),
// every thread owns 2 values of v, and threads 0..7 one beta each. Loaded a segment
// ahead into registers.
constexpr int TPT = SEG * DK / NT;     // tokens per thread in the staging
struct SegIn {
    uint16_t kk[TPT], qq[TPT];
    float sv[SEG];
    uint16_t vv[SEG * DV / NT];
    float beta;
};

__device__ __forceinline__ void load_segment(const PrefillArgs& P, int b, int h, int t, int L, int tid, int lr,
                                             SegIn& in) {
    const KArgs& A = P.base;
    const int H = A.H, T = P.T;
    const int quarter = tid / DK;
#pragma unroll
    for (int tt = 0; tt < SEG; ++tt) {
        in.sv[tt] = 0.f;
        if (tt < L) {
            const size_t base = ((size_t)b * T + t + tt) * H + h;
            in.sv[tt] = A.s_per_row ? P.s[base * DK + lr] : P.s[base];
        }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int tt = TPT * quarter + i;
        in.kk[i] = 0;
        in.qq[i] = 0;
        if (tt < L) {
            const size_t base = ((size_t)b * T + t + tt) * H + h;
            in.kk[i] = P.k[base * DK + lr];
            in.qq[i] = P.q[base * DK + lr];
        }
    }
#pragma unroll
    for (int n = 0; n < SEG * DV / NT; ++n) {
        const int i = tid + n * NT, tt = i / DV, j = i - tt * DV;
        in.vv[n] = tt < L ? P.v[(((size_t)b * T + t + tt) * H + h) * DV + j] : uint16_t(0);
    }
    in.beta = (tid < SEG && tid < L) ? P.beta[((size_t)b * T + t + tid) * H + h] : 0.f;
}

// length of the segment starting at t: up to min(chunk, 8) tokens, ending at the next
// write-back point or the last token
__device__ __forceinline__ int segment_length(int t, int T, int C, int chunk) {
    const int to_wb = C - (t % C);
    int L = chunk < SEG ? chunk : SEG;
    L = L < to_wb ? L : to_wb;
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
    const int col = 16 * wave + lc;                     // this lane's state column
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int k_hi = (KIND == WB_MIXED) ? A.k_hi : 0;
    const size_t code_base = (size_t)k_hi * DV * 2;
    const size_t meta_base = code_base + (size_t)(DK - k_hi) * DV;
    const int ub = A.bits;
    const double ustep = 1.0 / double(1 << (ub - 1));

    for (int i = tid; i < DK; i += NT) sm.perm[i] = (KIND == WB_MIXED) ? int(A.perm[h * DK + i]) : i;

    // ---- load and dequantize the stored state into the accumulator layout ----------
    f64x4 S[8];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
        double e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + lg + 4 * r;
            double x = 0.0;
            if (KIND == WB_FP32) {
                x = double(reinterpret_cast<const float*>(region)[row * DV + col]);
            } else if (KIND == WB_UNIFORM) {
                const int bit = (row * DV + col) * ub;
                const uint32_t byte = region[bit >> 3];
                int kap = int((byte >> (bit & 7)) & ((1u << ub) - 1));
                if (kap >= (1 << (ub - 1))) kap -= (1 << ub);
                x = double(kap) * ustep;
            } else if (KIND == WB_MIXED && row < k_hi) {
                x = f16d(reinterpret_cast<const uint16_t*>(region)[row * DV + col]);
            } else {
                const int qrow = row - k_hi;
                const uint32_t code = region[code_base + (size_t)qrow * DV + col];
                const uint32_t sz = *reinterpret_cast<const uint32_t*>(
                    region + meta_base + ((size_t)qrow * (DV / 32) + col / 32) * 4);
                x = f16d(sz >> 16) + double(code) * f16d(sz & 0xFFFFu);
            }
            e[r] = x;
        }
        S[rt] = f64x4{e[0], e[1], e[2], e[3]};
    }
    __syncthreads();

    const int T = P.T;
    const int my_lr = sm.perm[tid & (DK - 1)];
    SegIn nxt;
    load_segment(P, b, h, 0, segment_length(0, T, P.C, P.chunk), tid, my_lr, nxt);
    int t = 0;
    while (t < T) {
        const int L = segment_length(t, T, P.C, P.chunk);
        const bool write_back = ((t + L) % P.C == 0) || (t + L == T);
        const SegIn cur = nxt;

        // ---- stage inputs (physical row order) and the decay products ---------------
#pragma unroll
        for (int n = 0; n < SEG * DV / NT; ++n) {
            const int i = tid + n * NT, tt = i / DV, j = i - tt * DV;
            sm.v[tt][j] = bf16f(cur.vv[n]);
        }
        if (tid < SEG) sm.beta[tid] = double(cur.beta);
        {
            // thread t: row t % 128, tokens 2 (t / 128), +1
            const int p = tid & (DK - 1), quarter = tid / DK;
            double g[SEG];
            double acc = 0.0;
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                acc += double(cur.sv[tt]);
                g[tt] = acc;
            }
            const double decL = exp(-g[L - 1]);
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const int tt = TPT * quarter + i;
                const double kk = double(bf16f(cur.kk[i])), qq = double(bf16f(cur.qq[i]));
                const double dec = exp(-g[tt]);
                // e^{g}: reciprocal refined by two Newton steps (within an ulp)
                double inc = __builtin_amdgcn_rcp(dec);
                inc = fma(fma(-dec, inc, 1.0), inc, inc);
                inc = fma(fma(-dec, inc, 1.0), inc, inc);
                sm.u.st.khat[tt][pidx(p)] = kk * dec;
                sm.u.st.qhat[tt][pidx(p)] = qq * dec;
                sm.u.st.kqt[p][tt] = kk * dec;
                sm.u.st.kqt[p][SEG + tt] = qq * dec;
                sm.u.st.kbar[tt][pidx(p)] = kk * inc;
                sm.u.st.kbarL[tt][p] = kk * (inc * decL);
            }
            if (quarter == 0) sm.gl[p] = decL;
        }
        __syncthreads();
        // small Gram matrices: A[t][tau] = k^_t . k-_tau (tau < t), QK[t][tau] (tau <= t);
        // eight lanes per entry, 16 rows each
        {
            const int pair = tid >> 3, part = tid & 7;
            const int tt = pair / SEG, ta = pair - tt * SEG;
            double a = 0.0, q = 0.0;
            if (ta <= tt && tt < L) {
                const double* kh = &sm.u.st.khat[tt][17 * part];
                const double* qh = &sm.u.st.qhat[tt][17 * part];
                const double* kb = &sm.u.st.kbar[ta][17 * part];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    a = fma(kh[i], kb[i], a);
                    q = fma(qh[i], kb[i], q);
                }
            }
            a += mov_dpp_f64<0xB1>(a);      // xor 1
            q += mov_dpp_f64<0xB1>(q);
            a += mov_dpp_f64<0x4E>(a);      // xor 2
            q += mov_dpp_f64<0x4E>(q);
            a += mov_dpp_f64<0x141>(a);     // half mirror: the other quad of the 8 lanes
            q += mov_dpp_f64<0x141>(q);
            if (part == 0) {
                sm.A[tt][ta] = (ta < tt) ? a : 0.0;
                sm.QK[tt][ta] = (ta <= tt) ? q : 0.0;
            }
        }

        // ---- [k^; q^] S_0 on MFMA (16 x 16 per wave), rotated rows kept apart --------
        f64x4 accP = f64x4{0.0, 0.0, 0.0, 0.0}, accQ = accP;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const double a = sm.u.st.kqt[16 * rt + lg + 4 * r][lc];
                if (LY::rotated(rt))
                    accQ = __builtin_amdgcn_mfma_f64_16x16x4f64(a, S[rt][r], accQ, 0, 0, 0);
                else
                    accP = __builtin_amdgcn_mfma_f64_16x16x4f64(a, S[rt][r], accP, 0, 0, 0);
            }
        }
        // accumulator element (M = lg + 4r, column 16w + lc)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sm.u.st.ks[lg + 4 * r][col] = accP[r];
            if (LY::ROT) sm.u.st.ksq[lg + 4 * r][col] = accQ[r];
        }
        __syncthreads();
        if (LY::ROT) {
            // wave w transforms vectors 2w, 2w + 1 back from the rotated domain and adds
            // the unrotated part
#pragma unroll
            for (int vv = 0; vv < 2; ++vv) {
                const int m = 2 * wave + vv;
                double a0 = sm.u.st.ksq[m][lane], a1 = sm.u.st.ksq[m][lane + 64];
                wave_wht128(a0, a1, lane);
                sm.u.st.ks[m][lane] += a0;
                sm.u.st.ks[m][lane + 64] += a1;
            }
            __syncthreads();
        }

        // ---- per column: forward solve for w (threads 0..127) ------------------------
        if (tid < DV) {
            const int j = tid;
            double wv[SEG];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                double u = double(sm.v[tt][j]) - sm.u.st.ks[tt][j];
#pragma unroll
                for (int ta = 0; ta < tt; ++ta) u = fma(-sm.A[tt][ta], wv[ta], u);
                wv[tt] = sm.beta[tt] * u;
                sm.w[tt][j] = wv[tt];
            }
        }
        // inputs of the next segment (requested before this segment's output stores)
        if (t + L < T) load_segment(P, b, h, t + L, segment_length(t + L, T, P.C, P.chunk), tid, my_lr, nxt);
        __syncthreads();
        // ---- outputs o (threads 128..255) beside H w (waves 4..7) ----------------------
        if (tid >= DV && tid < 2 * DV) {
            const int j = tid - DV;
            double wv[SEG];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) wv[tt] = sm.w[tt][j];
#pragma unroll
            for (int tt = 0; tt < SEG; ++tt) {
                if (tt < L) {
                    double o = sm.u.st.ks[SEG + tt][j];
#pragma unroll
                    for (int ta = 0; ta <= tt; ++ta) o = fma(sm.QK[tt][ta], wv[ta], o);
                    P.o[(((size_t)b * T + t + tt) * H + h) * DV + j] = float(o);
                }
            }
        } else if (LY::ROT && wave >= 4) {
            // H w for the rotated rows: two vectors per wave
#pragma unroll
            for (int vv = 0; vv < 2; ++vv) {
                const int m = 2 * (wave - 4) + vv;
                double a0 = sm.w[m][lane], a1 = sm.w[m][lane + 64];
                wave_wht128(a0, a1, lane);
                sm.hw[m][lane] = a0;
                sm.hw[m][lane + 64] = a1;
            }
        }
        if (LY::ROT) __syncthreads();

        // ---- S_L = Gamma_L S_0 + sum_tau (Gamma_L k-_tau) w_tau^T  (MFMA, K = 8) ------
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            const double* wsrc = LY::rotated(rt) ? &sm.hw[0][0] : &sm.w[0][0];
            f64x4 c = S[rt];
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] *= sm.gl[16 * rt + lg + 4 * r];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int tok = 4 * kk + lg;
                const double a = sm.u.st.kbarL[tok][16 * rt + lc];
                const double bv = wsrc[tok * VS + col];
                c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, c, 0, 0, 0);
            }
            S[rt] = c;
        }

        // ---- write-back ---------------------------------------------------------------
        // Element-wise rows (the float16 rows of MIXED) round in registers. Rows with
        // per-block metadata (and UNIFORM rows, whose codes are packed across columns)
        // go through LDS in row-major order, up to four row tiles at a time: two
        // threads then round one 32-value row block (an INT8 block: extrema exchanged
        // between the pair, float16 metadata and levels), and the call's last
        // write-back stores its codes contiguously.
        if (write_back && KIND != WB_FP32) {
            const bool last = (t + L == T);
            if (KIND == WB_MIXED) {
                // row tile 0: physical rows 0..15, the float16 rows (k_hi = 16)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint16_t hb = f64_to_f16_bits(S[0][r]);
                    S[0][r] = f16d(hb);
                    if (last) reinterpret_cast<uint16_t*>(region)[(lg + 4 * r) * DV + col] = hb;
                }
            }
            constexpr int RT0 = KIND == WB_MIXED ? 1 : 0;
            __syncthreads();      // every wave is done with the staging area
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                const int g0 = RT0 + 4 * hv;                   // first row tile of this pass
                const int nrows = 16 * (8 - g0 < 4 ? 8 - g0 : 4);
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    if (RT0 + 4 * hv + rq < 8)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sm.u.wbuf[16 * rq + lg + 4 * r][widx(col)] = S[(RT0 + 4 * hv + rq) & 7][r];
                __syncthreads();
                // thread: row lrow, block cb (columns 32 cb .. +31), half hf (16 columns)
                const int lrow = tid >> 3, cb = (tid >> 1) & 3, hf = tid & 1;
                if (lrow < nrows) {
                    const int row = 16 * g0 + lrow;
                    double* rp = &sm.u.wbuf[lrow][33 * cb + 16 * hf];
                    double x[16];
#pragma unroll
                    for (int c = 0; c < 16; ++c) x[c] = rp[c];
                    const int col0 = 32 * cb + 16 * hf;
                    if (KIND == WB_UNIFORM) {
                        const double lo = -double(1 << (ub - 1)), hi = double((1 << (ub - 1)) - 1);
                        const double inv = double(1 << (ub - 1));
                        uint32_t wd[4] = {0, 0, 0, 0};           // 16 fields of ub <= 8 bits
#pragma unroll
                        for (int c = 0; c < 16; ++c) {
                            const double kv = fmin(fmax(rint(x[c] * inv), lo), hi);
                            x[c] = kv * ustep;
                            const int bit = c * ub;
                            wd[bit >> 5] |= (uint32_t(int(kv)) & ((1u << ub) - 1)) << (bit & 31);
                        }
                        if (last) {
                            // element (row, col) at bit ub (row DV + col): these 16 fields are
                            // 2 ub contiguous bytes, 2-byte aligned
                            uint16_t* dst = reinterpret_cast<uint16_t*>(region + ((row * DV + col0) * ub) / 8);
                            for (int i = 0; i < ub; ++i) dst[i] = uint16_t(wd[i >> 1] >> (16 * (i & 1)));
                        }
                    } else {
                        // affine INT8 block of 32 values: scale = f16((max - min) / 255) and
                        // zero = f16(min), each rounded once from float64; the level is
                        // (x - zero) / scale rounded to nearest (ties to even), clamped to
                        // [0, 255]: rounded by adding 1.5 * 2^52 (the integer lands in the
                        // low word), clamped as an integer, and rebuilt exactly from it
                        double mn = x[0], mx = x[0];
#pragma unroll
                        for (int c = 1; c < 16; ++c) {
                            mn = fmin(mn, x[c]);
                            mx = fmax(mx, x[c]);
                        }
                        mn = fmin(mn, mov_dpp_f64<0xB1>(mn));     // the pair's other half
                        mx = fmax(mx, mov_dpp_f64<0xB1>(mx));
                        // (a product with 1/255 in place of the quotient: the two differ by
                        // at most one float64 unit, which moves a float16 rounding only at
                        // a midpoint)
                        const uint16_t sb = f64_to_f16_bits(fmax(mx - mn, 0.0) * (1.0 / 255.0));
                        const uint16_t zb = f64_to_f16_bits(mn);
                        const double sc = f16d(sb), ze = f16d(zb);
                        uint32_t cw4[4] = {0, 0, 0, 0};
                        if (sc > 0.0) {
                            // reciprocal of the step refined by one Newton step (within a
                            // float64 unit of 1 / sc: a level moves only within ~1e-13 of a
                            // half-integer)
                            double inv = __builtin_amdgcn_rcp(sc);
                            inv = fma(fma(-sc, inv, 1.0), inv, inv);
                            constexpr double kM = 6755399441055744.0;          // 1.5 * 2^52
                            const int mhi = int(uint64_t(__double_as_longlong(kM)) >> 32);
#pragma unroll
                            for (int c = 0; c < 16; ++c) {
                                const double tm = (x[c] - ze) * inv + kM;
                                const int lev = min(max(int(uint32_t(__double_as_longlong(tm))), 0), 255);
                                x[c] = fma(__hiloint2double(mhi, lev) - kM, sc, ze);
                                cw4[c >> 2] |= uint32_t(lev) << (8 * (c & 3));
                            }
                        } else {
#pragma unroll
                            for (int c = 0; c < 16; ++c) x[c] = ze;
                        }
                        if (last) {
                            const int qrow = row - k_hi;
                            *reinterpret_cast<uint4*>(region + code_base + (size_t)qrow * DV + col0) =
                                make_uint4(cw4[0], cw4[1], cw4[2], cw4[3]);
                            if (hf == 0)
                                *reinterpret_cast<uint32_t*>(region + meta_base + ((size_t)qrow * (DV / 32) + cb) * 4) =
                                    uint32_t(sb) | (uint32_t(zb) << 16);
                        }
                    }
#pragma unroll
                    for (int c = 0; c < 16; ++c) rp[c] = x[c];
                }
                __syncthreads();
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    if (RT0 + 4 * hv + rq < 8)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            S[(RT0 + 4 * hv + rq) & 7][r] = sm.u.wbuf[16 * rq + lg + 4 * r][widx(col)];
                __syncthreads();
            }
        }
        if (KIND == WB_FP32 && write_back) {
            // identity write-back: the state continues from its float32 copy
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[rt][r] = double(float(S[rt][r]));
        }
        if (KIND == WB_FP32 && t + L == T) {
            // the stored float32 state
            float* dst = reinterpret_cast<float*>(region);
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * rt + lg + 4 * r) * DV + col] = float(S[rt][r]);
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
