// Fused decode write-back kernel and its import/export variants (gfx950, wave64).
//
// One workgroup owns one head state (b, h) and updates its region in place:
//   load + unpack codes -> dequantize -> decay -> u = k^T D S -> w = beta (v - u)
//   -> S' = D S + k w^T -> o = S'^T q (before quantization) -> metadata -> round
//   under the write-back rule -> pack -> store
// ([LBRS] "Accumulated readout error"; [DAMP] "Implementation": reconstruct the INT8
// channels, update in FP32, re-quantize, write back).
//
// Lane tile. Lane `tid` owns 8 rows x 8 consecutive columns: columns 8*cg .. 8*cg+7 with
// cg = tid % (dv/8), rows rg + (dk/8)*m for m = 0..7 with rg = tid / (dv/8). For
// dk = dv = 128 a wavefront covers 4 consecutive rows per m (512 contiguous bytes of
// INT8 codes per load instruction), and every lane holds exactly one of the first
// dk/8 physical rows (m = 0) -- the float16 rows of the mixed layout -- so the two
// storage tiers never diverge inside a wavefront.
//
// Hadamard rows stay in the rotated domain ([DAMP] "Key Points": the transform runs
// along the value dimension of each key channel): with Y = S H,
//   u = sum_P k_i a_i S_i + H sum_Q k_i a_i Y_i,   w = beta (v - u),
//   S_i' = a_i S_i + k_i w (float16 rows P),   Y_i' = a_i Y_i + k_i (H w) (rows Q),
//   o = sum_P q_i a_i S_i + H sum_Q q_i a_i Y_i + (q . k) w,
// so a step costs three 128-point vector transforms instead of one per row.
//
// Arithmetic. Layouts with Hadamard INT8 rows (HAD_INT8, MIXED) run the per-element
// path and the u/p reductions in float64: their stored codes must agree with a float64
// evaluation to within 1e-5 of a quantization step, and the float16 rows within 1e-5
// of a float16 spacing (~1e-8 relative), below float32 resolution. FP32, UNIFORM and
// BITALLOC run in float32.
#include <type_traits>

#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr double kInvSqrt128 = 0.08838834764831844055;  // 1/sqrt(128)

template <int DK, int DV>
struct Shape {
    static constexpr int NCG = DV / 8;                 // column groups (lanes per row)
    static constexpr int RS = DK / 8;                  // row groups (row stride between m)
    static constexpr int NACT = NCG * RS;              // lanes holding a tile
    static constexpr int NT = NACT < 64 ? 64 : NACT;   // workgroup size
    static constexpr int NW = NT / 64;
};

template <typename Real>
__device__ __forceinline__ Real rexp(Real x);
template <>
__device__ __forceinline__ double rexp<double>(double x) { return exp(x); }
template <>
__device__ __forceinline__ float rexp<float>(float x) { return expf(x); }

// 128-point orthonormal Walsh-Hadamard transform of one row held by 16 consecutive
// lanes (8 values each, lane cg holding elements 8*cg .. 8*cg+7).
template <typename Real>
__device__ __forceinline__ void row_wht128(Real v[8], int cg) {
#pragma unroll
    for (int span = 1; span < 8; span <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & span) == 0) {
                const Real a = v[i], b = v[i + span];
                v[i] = a + b;
                v[i + span] = a - b;
            }
        }
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const Real o = xor_shfl(v[i], d);
            v[i] = (cg & d) ? (o - v[i]) : (v[i] + o);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= Real(kInvSqrt128);
}

// 128-point transform of two vectors held by one wavefront, lane l holding elements
// l and l + 64 of each.
template <typename Real>
__device__ __forceinline__ void vec_wht128(Real& a0, Real& a1, int lane) {
    Real x = a0 + a1, y = a0 - a1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const Real ox = xor_shfl(x, d), oy = xor_shfl(y, d);
        x = (lane & d) ? (ox - x) : (x + ox);
        y = (lane & d) ? (oy - y) : (y + oy);
    }
    a0 = x * Real(kInvSqrt128);
    a1 = y * Real(kInvSqrt128);
}

template <int DK, int DV, int KIND>
struct Smem {
    static constexpr bool ROT = KIND == WB_HAD_INT8 || KIND == WB_MIXED;
    using Real = typename std::conditional<ROT, double, float>::type;
    static constexpr int NQ = ROT ? 4 : 2;             // reduced quantities: uP, pP (, uQ, pQ)
    // BITALLOC (and HEADALLOC, run by the same instantiations): codes up to 8 bits per
    // value, then the larger of the two metadata blocks
    static constexpr int HA_META = 3 * (DK / 32) * DV + 16;
    static constexpr int BA_WORDS = (KIND == WB_BITALLOC) ? (DK * DV + (HA_META > 3 * DK ? HA_META : 3 * DK)) / 4 + 4 : 1;
    static constexpr int HA_N = (KIND == WB_BITALLOC) ? (DK / 32) * DV : 1;
    Real k[DK], q[DK], a[DK];
    Real red[Shape<DK, DV>::NW][NQ][DV];
    Real vec[NQ][DV];
    Real w[DV], wr[DV];
    int perm[DK];
    // BITALLOC: the region's bytes, and per-row width, fit, byte offset and Delta
    uint32_t reg[BA_WORDS];
    int width[KIND == WB_BITALLOC ? DK : 1];
    int fit[KIND == WB_BITALLOC ? DK : 1];
    int off[KIND == WB_BITALLOC ? DK : 1];
    float delta[KIND == WB_BITALLOC ? DK : 1];
    int used;                       // BITALLOC code bytes of the head (sum of widths * DV / 8)
    // HEADALLOC: group maxima per wavefront, then the groups' Delta
    float gred[KIND == WB_BITALLOC ? 4 : 1][HA_N];
    float gdelta[HA_N];
};

template <int KIND, int MODE, int OP, int DK, int DV>
__global__ void __launch_bounds__((Shape<DK, DV>::NT)) wb_kernel(const KArgs A) {
    using Sh = Shape<DK, DV>;
    using SM = Smem<DK, DV, KIND>;
    using Real = typename SM::Real;
    constexpr bool ROT = SM::ROT;
    constexpr int NCG = Sh::NCG, RS = Sh::RS, NT = Sh::NT;
    constexpr int EMODE = (OP == OP_IMPORT) ? WB_RTN : MODE;    // import rounds to nearest
    constexpr bool MEM = MODE == WB_DIR || MODE == WB_RESQ;        // temporal memory (UNIFORM)
    constexpr bool USE_SIDE = (MODE == WB_EF || MEM) && (KIND != WB_FP32);
    static_assert(!MEM || KIND == WB_UNIFORM, "temporal-memory rules are defined on the uniform grid");

    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int head = blockIdx.x;
    const int b = head / A.H, h = head - b * A.H;
    const bool act = tid < Sh::NACT;
    const int cg = tid % NCG, rg = act ? tid / NCG : 0;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int mhi = (KIND == WB_MIXED) ? A.k_hi / RS : 0;     // m < mhi: float16 rows

    // ---- per-head vectors, in physical row order -------------------------------
    for (int i = tid; i < DK; i += NT) {
        const int lr = (KIND == WB_MIXED) ? int(A.perm[h * DK + i]) : i;
        sm.perm[i] = lr;
        if (OP == OP_STEP) {
            sm.k[i] = Real(A.k[(size_t)head * DK + lr]);
            sm.q[i] = Real(A.q[(size_t)head * DK + lr]);
            const float sv = A.s_per_row ? A.s[(size_t)head * DK + lr] : A.s[head];
            sm.a[i] = rexp<Real>(-Real(sv));
            if (KIND == WB_BITALLOC && A.est)
                ema_fold_row(A.est + (size_t)head * est_stride(DK), DK, i, sv, A.beta[head], A.k[(size_t)head * DK + i]);
        }
    }

    // ---- BITALLOC: stage the region in LDS, derive widths and row offsets --------
    if (KIND == WB_BITALLOC) {
        // Delta and meta follow the code area (A.code_cap bytes); under the per-head
        // budget the codes fill it and the whole region is staged at once, under the
        // layer budget the metadata is staged first and the codes up to the head's
        // last row after the widths are known (below)
        const int code_bytes = A.code_cap;
        const int total = code_bytes + (A.head_unit ? SM::HA_META : 3 * DK);
        const uint4* src = reinterpret_cast<const uint4*>(region);
        for (int i = A.layer ? code_bytes / 16 + tid : tid; i * 16 < total; i += NT) {
            reinterpret_cast<uint4*>(sm.reg)[i] = src[i];
        }
        __syncthreads();
        const uint8_t* bytes = reinterpret_cast<const uint8_t*>(sm.reg);
        if (wave == 0) {
            constexpr int RPL = (DK + 63) / 64;     // rows per lane in the scan
            int local = 0;
            int wv[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int row = lane * RPL + r;
                int wdt = 0;
                if (row < DK && A.head_unit) {
                    // one width for the head; the group scales stay in the staged bytes
                    wdt = int(bytes[code_bytes + 3 * (DK / 32) * DV]) + 1;
                    sm.width[row] = wdt;
                } else if (row < DK) {
                    const int meta = bytes[code_bytes + 2 * DK + row];
                    wdt = (meta & 7) + 1;
                    sm.width[row] = wdt;
                    sm.fit[row] = meta >> 4;
                    const uint32_t db = uint32_t(bytes[code_bytes + 2 * row]) |
                                        (uint32_t(bytes[code_bytes + 2 * row + 1]) << 8);
                    sm.delta[row] = f16_bits_to_f32(db);
                }
                wv[r] = wdt * (DV / 8);
                local += wv[r];
            }
            int incl = local;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            int run = incl - local;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int row = lane * RPL + r;
                if (row < DK) sm.off[row] = run;
                run += wv[r];
            }
            if (lane == 63) sm.used = incl;
        }
        if (A.layer) {
            __syncthreads();
            const int used = sm.used;
            for (int i = tid; i * 16 < used; i += NT) reinterpret_cast<uint4*>(sm.reg)[i] = src[i];
        }
    }
    __syncthreads();

    // ---- load the lane's tile (stored domain) ------------------------------------
    Real x[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[m][c] = Real(0);
    }
    if (act) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = rg + RS * m;
            if (OP == OP_IMPORT) {
                const float* src = A.S_in + ((size_t)head * DK + sm.perm[row]) * DV + 8 * cg;
                const float4 v0 = reinterpret_cast<const float4*>(src)[0];
                const float4 v1 = reinterpret_cast<const float4*>(src)[1];
                const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int c = 0; c < 8; ++c) x[m][c] = Real(f[c]);
                if (ROT && (KIND == WB_HAD_INT8 || m >= mhi)) row_wht128<Real>(x[m], cg);
                continue;
            }
            if (KIND == WB_FP32) {
                const float* src = reinterpret_cast<const float*>(region) + row * DV + 8 * cg;
                const float4 v0 = reinterpret_cast<const float4*>(src)[0];
                const float4 v1 = reinterpret_cast<const float4*>(src)[1];
                const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int c = 0; c < 8; ++c) x[m][c] = Real(f[c]);
            } else if (KIND == WB_UNIFORM) {
                const int B = A.bits;
                const Real step = Real(1) / Real(1 << (B - 1));
                const size_t boff = ((size_t)row * DV / 8 + cg) * B;   // 8 fields = B bytes
                uint64_t fld;
                if (B == 2) fld = *reinterpret_cast<const uint16_t*>(region + boff);
                else if (B == 4) fld = *reinterpret_cast<const uint32_t*>(region + boff);
                else fld = *reinterpret_cast<const uint64_t*>(region + boff);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    int kap = int((fld >> (c * B)) & ((1u << B) - 1));
                    if (kap >= (1 << (B - 1))) kap -= (1 << B);
                    x[m][c] = Real(kap) * step;
                }
            } else if (KIND == WB_MIXED && m < mhi) {
                const uint4 raw = *reinterpret_cast<const uint4*>(region + ((size_t)row * DV + 8 * cg) * 2);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    x[m][c] = Real(f16_bits_to_f32((w4[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu));
            } else if (ROT) {
                const int k_hi = (KIND == WB_MIXED) ? A.k_hi : 0;
                const int qrow = row - k_hi;
                const int ib = A.int_bits;                // 8, or 4: codes two a byte
                const size_t code_base = (size_t)k_hi * DV * 2;
                const size_t meta_base = code_base + (size_t)(DK - k_hi) * DV * ib / 8;
                const uint8_t* cp = region + code_base + ((size_t)qrow * DV + 8 * cg) * ib / 8;
                uint2 raw;
                if (ib == 8) raw = *reinterpret_cast<const uint2*>(cp);
                else raw = make_uint2(*reinterpret_cast<const uint32_t*>(cp), 0u);
                const int nb = DV / A.block;
                const int g = (8 * cg) / A.block;
                const uint32_t sz = *reinterpret_cast<const uint32_t*>(region + meta_base + ((size_t)qrow * nb + g) * 4);
                const Real scale = Real(f16_bits_to_f32(sz & 0xFFFFu));
                const Real zero = Real(f16_bits_to_f32(sz >> 16));
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t code = ib == 8 ? ((c < 4 ? raw.x : raw.y) >> ((c & 3) * 8)) & 0xFFu
                                                  : (raw.x >> (c * 4)) & 0xFu;
                    x[m][c] = zero + Real(code) * scale;
                }
            } else if (KIND == WB_BITALLOC) {
                const int bw = sm.width[row];
                const int n = (1 << (bw - 1)) - 1;
                const int off = sm.off[row] + cg * bw;
                const int wi = off >> 2, sh = (off & 3) * 8;
                const uint64_t lo = uint64_t(sm.reg[wi]) | (uint64_t(sm.reg[wi + 1]) << 32);
                uint64_t fld = lo >> sh;
                if (sh) fld |= uint64_t(sm.reg[wi + 2]) << (64 - sh);
                const float dl = sm.delta[row];
                const uint64_t mask = (1ull << bw) - 1;
                // HEADALLOC: the scale of (row / 32, column)
                const uint16_t* gs = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sm.reg) +
                                                                       A.code_cap) + (row >> 5) * DV + 8 * cg;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int field = int((fld >> (c * bw)) & mask);
                    const int kap = bw == 1 ? 2 * field - 1 : field - n;   // one-bit rows: -1, +1
                    x[m][c] = Real(float(kap) * (A.head_unit ? f16_bits_to_f32(gs[c]) : dl));
                }
            }
        }
    }

    // ---- export: back to the original domain, logical order ---------------------
    if (OP == OP_EXPORT) {
        if (act) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int row = rg + RS * m;
                if (ROT && (KIND == WB_HAD_INT8 || m >= mhi)) row_wht128<Real>(x[m], cg);
                float* dst = A.S_out + ((size_t)head * DK + sm.perm[row]) * DV + 8 * cg;
                reinterpret_cast<float4*>(dst)[0] = make_float4(float(x[m][0]), float(x[m][1]), float(x[m][2]), float(x[m][3]));
                reinterpret_cast<float4*>(dst)[1] = make_float4(float(x[m][4]), float(x[m][5]), float(x[m][6]), float(x[m][7]));
            }
        }
        return;
    }

    if (OP == OP_STEP) {
        // ---- u, p partial sums over the lane's rows -----------------------------
        Real acc[SM::NQ][8];
#pragma unroll
        for (int qn = 0; qn < SM::NQ; ++qn)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[qn][c] = Real(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = rg + RS * m;
            const Real ka = sm.k[row] * sm.a[row];
            const Real qa = sm.q[row] * sm.a[row];
            const bool rot = ROT && (KIND == WB_HAD_INT8 || m >= mhi);
            const int base = rot ? 2 : 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (rot) {
                    acc[SM::NQ - 2][c] += ka * x[m][c];
                    acc[SM::NQ - 1][c] += qa * x[m][c];
                } else {
                    acc[0][c] += ka * x[m][c];
                    acc[1][c] += qa * x[m][c];
                }
            }
            (void)base;
        }
        // reduce over the row groups of this wavefront, then across wavefronts
#pragma unroll
        for (int qn = 0; qn < SM::NQ; ++qn)
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int d = NCG; d < 64; d <<= 1) acc[qn][c] += xor_shfl(acc[qn][c], d);
        if (act && lane < NCG) {
#pragma unroll
            for (int qn = 0; qn < SM::NQ; ++qn)
#pragma unroll
                for (int c = 0; c < 8; ++c) sm.red[wave][qn][8 * cg + c] = acc[qn][c];
        }
        __syncthreads();
        for (int i = tid; i < SM::NQ * DV; i += NT) {
            const int qn = i / DV, j = i - qn * DV;
            Real sum = Real(0);
#pragma unroll
            for (int w = 0; w < Sh::NW; ++w) sum += sm.red[w][qn][j];
            sm.vec[qn][j] = sum;
        }
        __syncthreads();

        // ---- vector phase: u, w, H w, o (one wavefront) -------------------------
        if (wave == 0) {
            Real qk = Real(0);
            for (int i = lane; i < DK; i += 64) qk += sm.q[i] * sm.k[i];
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) qk += xor_shfl(qk, d);
            const Real beta = Real(A.beta[head]);
            if constexpr (ROT) {
                // DV == 128: lane holds elements lane and lane + 64
                Real uq0 = sm.vec[2][lane], uq1 = sm.vec[2][lane + 64];
                Real pq0 = sm.vec[3][lane], pq1 = sm.vec[3][lane + 64];
                vec_wht128<Real>(uq0, uq1, lane);
                vec_wht128<Real>(pq0, pq1, lane);
                const Real u0 = sm.vec[0][lane] + uq0, u1 = sm.vec[0][lane + 64] + uq1;
                const Real p0 = sm.vec[1][lane] + pq0, p1 = sm.vec[1][lane + 64] + pq1;
                const Real w0 = beta * (Real(A.v[(size_t)head * DV + lane]) - u0);
                const Real w1 = beta * (Real(A.v[(size_t)head * DV + lane + 64]) - u1);
                A.o[(size_t)head * DV + lane] = float(p0 + qk * w0);
                A.o[(size_t)head * DV + lane + 64] = float(p1 + qk * w1);
                sm.w[lane] = w0;
                sm.w[lane + 64] = w1;
                Real r0 = w0, r1 = w1;
                vec_wht128<Real>(r0, r1, lane);
                sm.wr[lane] = r0;
                sm.wr[lane + 64] = r1;
            } else {
                for (int j = lane; j < DV; j += 64) {
                    const Real u = sm.vec[0][j];
                    const Real p = sm.vec[1][j];
                    const Real w = beta * (Real(A.v[(size_t)head * DV + j]) - u);
                    A.o[(size_t)head * DV + j] = float(p + qk * w);
                    sm.w[j] = w;
                }
            }
        }
        __syncthreads();

        // ---- update: S' = D S + k w^T (rotated rows take H w) --------------------
        if (act) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int row = rg + RS * m;
                const Real am = sm.a[row], km = sm.k[row];
                const bool rot = ROT && (KIND == WB_HAD_INT8 || m >= mhi);
                const Real* wv = rot ? sm.wr : sm.w;
#pragma unroll
                for (int c = 0; c < 8; ++c) x[m][c] = am * x[m][c] + km * wv[8 * cg + c];
            }
        }
    }

    // ---- requantize and store ------------------------------------------------------
    if (KIND == WB_BITALLOC) {
        // clear the code area of the LDS copy; codes are OR-ed in, then copied out
        __syncthreads();
        const int code_words = sm.used / 4;
        for (int i = tid; i < code_words; i += NT) sm.reg[i] = 0u;
        __syncthreads();
        if constexpr (KIND == WB_BITALLOC && DK == 128) if (A.head_unit) {
            // HEADALLOC: Delta of each group (32 rows of one column) from its maximum and
            // its stored fit index. Rows rg + 16 m: the lane's rows of group g are m = 2g,
            // 2g + 1; the group's other rows sit in the lanes 16 and 32 apart and in the
            // other wavefronts.
            constexpr int NGR = DK / 32;
            float gm[NGR][8];
#pragma unroll
            for (int g = 0; g < NGR; ++g)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float v = fmaxf(fabsf(float(x[2 * g][c])), fabsf(float(x[2 * g + 1][c])));
                    auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                    v = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
                    auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                    gm[g][c] = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
                }
            if (lane < 16) {
#pragma unroll
                for (int g = 0; g < NGR; ++g)
#pragma unroll
                    for (int c = 0; c < 8; ++c) sm.gred[wave][g * DV + 8 * cg + c] = gm[g][c];
            }
            __syncthreads();
            const int n = (1 << (sm.width[0] - 1)) - 1;
            uint8_t* lb = reinterpret_cast<uint8_t*>(sm.reg);
            for (int i = tid; i < NGR * DV; i += NT) {
                const float R = fmaxf(fmaxf(sm.gred[0][i], sm.gred[1][i]), fmaxf(sm.gred[2][i], sm.gred[3][i]));
                const double f = 0.25 + double(lb[A.code_cap + 2 * NGR * DV + i]) / 20.0;
                const uint16_t dbits = f64_to_f16_bits(f * double(R) / double(n));
                sm.gdelta[i] = f16_bits_to_f32(dbits);
                reinterpret_cast<uint16_t*>(lb + A.code_cap)[i] = dbits;      // for the write-back
            }
            __syncthreads();
        }
    }
    // write activity of this lane (UNIFORM decode steps with counters attached): dead-zone,
    // level changes, votes, triggers, sub-threshold writes, same-sign and opposite-sign
    // vote transitions, runs started
    uint32_t nact[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (act) {
        const uint32_t bh = uint32_t(head);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = rg + RS * m;
            uint32_t r16[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const bool hi_row = (KIND == WB_MIXED && m < mhi);
            // the side value of the lane's 8 elements of this row (residual, counter or
            // residual value), read here rather than with the codes so that it does not
            // hold registers through the contractions
            float em[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (USE_SIDE && OP == OP_STEP && !hi_row) {
                const float* src = A.side + ((size_t)head * DK + row) * DV + 8 * cg;
                const float4 v0 = reinterpret_cast<const float4*>(src)[0];
                const float4 v1 = reinterpret_cast<const float4*>(src)[1];
                em[0] = v0.x; em[1] = v0.y; em[2] = v0.z; em[3] = v0.w;
                em[4] = v1.x; em[5] = v1.y; em[6] = v1.z; em[7] = v1.w;
            }
            if (EMODE == WB_SR && KIND != WB_FP32 && !hi_row) sr_draws8(A.seed, bh, A.t, row, cg, r16);
            float en[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (KIND == WB_FP32) {
                float* dst = reinterpret_cast<float*>(region) + row * DV + 8 * cg;
                reinterpret_cast<float4*>(dst)[0] = make_float4(float(x[m][0]), float(x[m][1]), float(x[m][2]), float(x[m][3]));
                reinterpret_cast<float4*>(dst)[1] = make_float4(float(x[m][4]), float(x[m][5]), float(x[m][6]), float(x[m][7]));
                continue;
            } else if (KIND == WB_UNIFORM) {
                const int B = A.bits;
                const Real step = Real(1) / Real(1 << (B - 1));
                const Real inv_step = Real(1 << (B - 1));
                const int lo = -(1 << (B - 1)), hi = (1 << (B - 1)) - 1;
                const size_t boff = ((size_t)row * DV / 8 + cg) * B;
                // levels entering the step (still stored: this lane writes its fields below)
                const bool track = OP == OP_STEP && (MEM || A.activity != nullptr);
                uint64_t prev = 0;
                if (track) {
                    if (B == 2) prev = *reinterpret_cast<const uint16_t*>(region + boff);
                    else if (B == 4) prev = *reinterpret_cast<const uint32_t*>(region + boff);
                    else prev = *reinterpret_cast<const uint64_t*>(region + boff);
                }
                // vote state of the previous step, one byte per element: 0 none, 1 / 2 a
                // positive / negative vote with its run open, +4 when the run closed
                const bool count = OP == OP_STEP && A.activity != nullptr;
                uint8_t* vptr = count ? A.votes + ((size_t)head * DK + row) * DV + 8 * cg : nullptr;
                const uint64_t vprev = count ? *reinterpret_cast<const uint64_t*>(vptr) : 0ull;
                uint64_t vnew = 0;
                uint64_t fld = 0;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    int kp = 0;
                    if (track) {
                        kp = int((prev >> (c * B)) & ((1u << B) - 1));
                        if (kp >= (1 << (B - 1))) kp -= (1 << B);
                    }
                    const Real h = x[m][c];
                    const Real dlt = h - Real(kp) * step;
                    const Real ad = fabs(dlt);
                    const bool vote = ad > Real(0.125) * step && ad < Real(0.5) * step;
                    int kap;
                    bool trig = false;
                    if constexpr (EMODE == WB_RESQ) {
                        // error feedback with the residual kept on the k-bit grid
                        const Real target = h + Real(em[c]);
                        kap = int(fmin(fmax(rint(target * inv_step), Real(lo)), Real(hi)));
                        const Real r = fmin(fmax(target - Real(kap) * step, -step), step);
                        const int hk = 1 << (A.mem_bits - 1);
                        const Real sub = step / Real(hk);
                        const Real j = fmin(fmax(rint(r / sub), Real(-hk)), Real(hk - 1));
                        en[c] = float(j * sub);
                    } else if constexpr (EMODE == WB_DIR) {
                        // direction memory: counter in the side buffer
                        const int near = int(fmin(fmax(rint(h * inv_step), Real(lo)), Real(hi)));
                        const float cnt = em[c];
                        if (near != kp) {
                            kap = near;
                            en[c] = 0.f;
                        } else if (vote) {
                            const int sg = dlt > Real(0) ? 1 : -1;
                            const float c2 = cnt + float(sg);
                            trig = fabsf(c2) >= float(1 << (A.mem_bits - 1));
                            kap = trig ? min(max(kp + sg, lo), hi) : kp;
                            en[c] = trig ? 0.f : c2;
                        } else {
                            kap = kp;
                            en[c] = cnt;
                        }
                    } else {
                        kap = round_rule<EMODE, Real>(h, Real(em[c]), step, Real(0), lo, hi, r16[c], &en[c]);
                    }
                    if (count) {
                        const bool dead = Real(2) * ad < step, change = kap != kp;
                        const uint32_t vp = uint32_t(vprev >> (8 * c)) & 0xFFu;
                        const uint32_t sg = vote ? (dlt > Real(0) ? 1u : 2u) : 0u;
                        nact[0] += dead;
                        nact[1] += change;
                        nact[2] += vote;
                        nact[3] += trig;
                        nact[4] += dead && change;
                        nact[5] += vote && (vp & 3u) == sg;
                        nact[6] += vote && (vp & 3u) != 0u && (vp & 3u) != sg;
                        nact[7] += vote && vp != sg;
                        vnew |= uint64_t(sg | ((vote && (change || trig)) ? 4u : 0u)) << (8 * c);
                    }
                    fld |= uint64_t(uint32_t(kap) & ((1u << B) - 1)) << (c * B);
                }
                if (count) *reinterpret_cast<uint64_t*>(vptr) = vnew;
                if (B == 2) *reinterpret_cast<uint16_t*>(region + boff) = uint16_t(fld);
                else if (B == 4) *reinterpret_cast<uint32_t*>(region + boff) = uint32_t(fld);
                else *reinterpret_cast<uint64_t*>(region + boff) = fld;
            } else if (hi_row) {
                uint32_t w4[4] = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 8; ++c) w4[c >> 1] |= uint32_t(to_f16_bits<Real>(x[m][c])) << ((c & 1) * 16);
                *reinterpret_cast<uint4*>(region + ((size_t)row * DV + 8 * cg) * 2) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                continue;
            } else if (ROT) {
                const int k_hi = (KIND == WB_MIXED) ? A.k_hi : 0;
                const int qrow = row - k_hi;
                const int ib = A.int_bits;
                const int top = (1 << ib) - 1;            // 255 or 15
                const size_t code_base = (size_t)k_hi * DV * 2;
                const size_t meta_base = code_base + (size_t)(DK - k_hi) * DV * ib / 8;
                const int LB = A.block / 8;               // lanes per block
                Real mn = x[m][0], mx = x[m][0];
#pragma unroll
                for (int c = 1; c < 8; ++c) {
                    mn = fmin(mn, x[m][c]);
                    mx = fmax(mx, x[m][c]);
                }
                for (int d = 1; d < LB; d <<= 1) {
                    mn = fmin(mn, xor_shfl(mn, d));
                    mx = fmax(mx, xor_shfl(mx, d));
                }
                const Real spre = fmax(mx - mn, Real(0)) / Real(top);
                const uint16_t sbits = to_f16_bits<Real>(spre);
                const uint16_t zbits = to_f16_bits<Real>(mn);
                const Real scale = Real(f16_bits_to_f32(sbits));
                const Real zero = Real(f16_bits_to_f32(zbits));
                uint32_t lo4 = 0, hi4 = 0;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int code = round_rule<EMODE, Real>(x[m][c], Real(em[c]), scale, zero, 0, top, r16[c], &en[c]);
                    if (ib == 4) lo4 |= uint32_t(code) << (c * 4);
                    else if (c < 4) lo4 |= uint32_t(code) << (c * 8);
                    else hi4 |= uint32_t(code) << ((c - 4) * 8);
                }
                uint8_t* cp = region + code_base + ((size_t)qrow * DV + 8 * cg) * ib / 8;
                if (ib == 8) *reinterpret_cast<uint2*>(cp) = make_uint2(lo4, hi4);
                else *reinterpret_cast<uint32_t*>(cp) = lo4;
                if ((cg % LB) == 0) {
                    const int nb = DV / A.block;
                    const int g = (8 * cg) / A.block;
                    *reinterpret_cast<uint32_t*>(region + meta_base + ((size_t)qrow * nb + g) * 4) =
                        uint32_t(sbits) | (uint32_t(zbits) << 16);
                }
            } else if (KIND == WB_BITALLOC) {
                const int bw = sm.width[row];
                const int n = (1 << (bw - 1)) - 1;
                uint16_t dbits = 0;
                float dl = 0.f;
                if (bw == 1) {
                    // one-bit row: Delta = f16(mean |x|); the rule on -Delta + k' 2 Delta
                    double sa = 0.0;
#pragma unroll
                    for (int c = 0; c < 8; ++c) sa += fabs(double(x[m][c]));
#pragma unroll
                    for (int d = 1; d < NCG; d <<= 1) sa += xor_shfl(sa, d);
                    dbits = f64_to_f16_bits(sa / double(DV));
                    dl = f16_bits_to_f32(dbits);
                } else if (!A.head_unit) {
                    float R = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) R = fmaxf(R, fabsf(float(x[m][c])));
#pragma unroll
                    for (int d = 1; d < NCG; d <<= 1) R = fmaxf(R, xor_shfl(R, d));
                    const double f = 0.25 + double(sm.fit[row]) / 20.0;
                    dbits = f64_to_f16_bits(f * double(R) / double(n));
                    dl = f16_bits_to_f32(dbits);
                }
                uint64_t fld = 0;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float dc = A.head_unit ? sm.gdelta[(row >> 5) * DV + 8 * cg + c] : dl;
                    if (bw == 1) {
                        const int k1 = round_rule<EMODE, float>(float(x[m][c]), em[c], 2.f * dl, -dl, 0, 1, r16[c], &en[c]);
                        fld |= uint64_t(uint32_t(k1)) << c;
                        continue;
                    }
                    const int kap = round_rule<EMODE, float>(float(x[m][c]), em[c], dc, 0.f, -n, n, r16[c], &en[c]);
                    fld |= uint64_t(uint32_t(kap + n)) << (c * bw);
                }
                const int off = sm.off[row] + cg * bw;
                const int wi = off >> 2, sh = (off & 3) * 8;
                const uint64_t lo = fld << sh;
                atomicOr(&sm.reg[wi], uint32_t(lo));
                atomicOr(&sm.reg[wi + 1], uint32_t(lo >> 32));
                if (sh) {
                    const uint32_t top = uint32_t(fld >> (64 - sh));
                    if (top) atomicOr(&sm.reg[wi + 2], top);
                }
                if (cg == 0 && !A.head_unit) {
                    reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(sm.reg) + A.code_cap)[row] = dbits;
                }
            }
            if (USE_SIDE) {
                float* dst = A.side + ((size_t)head * DK + row) * DV + 8 * cg;
                reinterpret_cast<float4*>(dst)[0] = make_float4(en[0], en[1], en[2], en[3]);
                reinterpret_cast<float4*>(dst)[1] = make_float4(en[4], en[5], en[6], en[7]);
            }
        }
    }
    if (KIND == WB_UNIFORM && OP == OP_STEP && A.activity != nullptr) {
        // sum over the wavefront, one atomic add per counter and wavefront
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) nact[i] += __shfl_xor(nact[i], d, 64);
        }
        if (lane == 0) {
            uint32_t* ctr = A.activity + (size_t)head * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) atomicAdd(ctr + i, nact[i]);
        }
    }
    if (KIND == WB_BITALLOC) {
        __syncthreads();
        // codes up to the head's last row, then Delta (meta unchanged)
        uint4* dst = reinterpret_cast<uint4*>(region);
        const uint4* lds = reinterpret_cast<const uint4*>(sm.reg);
        const int used = sm.used;
        for (int i = tid; i * 16 < used; i += NT) dst[i] = lds[i];
        const int delta_bytes = A.head_unit ? 2 * (DK / 32) * DV : 2 * DK;
        for (int i = tid; i * 16 < delta_bytes; i += NT) dst[A.code_cap / 16 + i] = lds[A.code_cap / 16 + i];
    }
}

template <int KIND, int MODE, int OP, int DK, int DV>
hipError_t launch_one(const KArgs& a, int heads, hipStream_t stream) {
    hipLaunchKernelGGL((wb_kernel<KIND, MODE, OP, DK, DV>), dim3(heads), dim3(Shape<DK, DV>::NT), 0,
                       stream, a);
    return hipGetLastError();
}

template <int KIND, int OP, int DK, int DV>
hipError_t launch_mode(int mode, const KArgs& a, int heads, hipStream_t stream) {
    if (KIND == WB_FP32 || OP == OP_EXPORT) return launch_one<KIND, WB_RTN, OP, DK, DV>(a, heads, stream);
    if constexpr (KIND == WB_UNIFORM) {
        if (mode == WB_DIR) return launch_one<KIND, WB_DIR, OP, DK, DV>(a, heads, stream);
        if (mode == WB_RESQ) return launch_one<KIND, WB_RESQ, OP, DK, DV>(a, heads, stream);
    }
    switch (mode) {
        case WB_RTN: return launch_one<KIND, WB_RTN, OP, DK, DV>(a, heads, stream);
        case WB_SR: return launch_one<KIND, WB_SR, OP, DK, DV>(a, heads, stream);
        default: return launch_one<KIND, WB_EF, OP, DK, DV>(a, heads, stream);
    }
}

template <int KIND, int DK, int DV>
hipError_t launch_op(int op, int mode, const KArgs& a, int heads, hipStream_t stream) {
    switch (op) {
        case OP_STEP: return launch_mode<KIND, OP_STEP, DK, DV>(mode, a, heads, stream);
        case OP_IMPORT: return launch_mode<KIND, OP_IMPORT, DK, DV>(mode, a, heads, stream);
        default: return launch_mode<KIND, OP_EXPORT, DK, DV>(mode, a, heads, stream);
    }
}

__global__ void fill_kernel(uint8_t* dst, size_t n, uint4 p0, int period) {
    const uint8_t* pat = reinterpret_cast<const uint8_t*>(&p0);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = pat[i % period];
}

// codes of the zero state on [0, code_bytes) (the rest of the code area keeps the zero
// fill), Delta = 0 and the meta bytes after the code area of `cap` bytes
__global__ void init_bitalloc_kernel(uint8_t* state, uint64_t stride, int code_bytes, int cap, uint4 p0,
                                     int period, int dk, uint8_t meta) {
    const uint8_t* pat = reinterpret_cast<const uint8_t*>(&p0);
    uint8_t* reg = state + (size_t)blockIdx.x * stride;
    for (int i = threadIdx.x; i < code_bytes; i += blockDim.x) reg[i] = pat[i % period];
    for (int i = threadIdx.x; i < 2 * dk; i += blockDim.x) reg[cap + i] = 0;
    for (int i = threadIdx.x; i < dk; i += blockDim.x) reg[cap + 2 * dk + i] = meta;
}

}  // namespace

hipError_t launch_init_bitalloc(uint8_t* state, uint64_t stride, int heads, int code_bytes, int cap,
                                const uint8_t* pattern, int period, int dk, uint8_t meta, hipStream_t stream) {
    uint4 p{0, 0, 0, 0};
    uint8_t* pb = reinterpret_cast<uint8_t*>(&p);
    for (int i = 0; i < period && i < 16; ++i) pb[i] = pattern[i];
    hipLaunchKernelGGL(init_bitalloc_kernel, dim3(heads), dim3(256), 0, stream, state, stride, code_bytes, cap, p,
                       period, dk, meta);
    return hipGetLastError();
}

__global__ void init_headalloc_kernel(uint8_t* state, uint64_t stride, int code_bytes, int cap, uint4 p0,
                                      int period, int groups, uint8_t wbyte) {
    const uint8_t* pat = reinterpret_cast<const uint8_t*>(&p0);
    uint8_t* reg = state + (size_t)blockIdx.x * stride;
    for (int i = threadIdx.x; i < code_bytes; i += blockDim.x) reg[i] = pat[i % period];
    for (int i = threadIdx.x; i < 2 * groups; i += blockDim.x) reg[cap + i] = 0;
    for (int i = threadIdx.x; i < groups; i += blockDim.x) reg[cap + 2 * groups + i] = 15;
    if (threadIdx.x == 0) reg[cap + 3 * groups] = wbyte;
}

hipError_t launch_init_headalloc(uint8_t* state, uint64_t stride, int heads, int code_bytes, int cap,
                                 const uint8_t* pattern, int period, int groups, uint8_t wbyte, hipStream_t stream) {
    uint4 p{0, 0, 0, 0};
    uint8_t* pb = reinterpret_cast<uint8_t*>(&p);
    for (int i = 0; i < period && i < 16; ++i) pb[i] = pattern[i];
    hipLaunchKernelGGL(init_headalloc_kernel, dim3(heads), dim3(256), 0, stream, state, stride, code_bytes, cap, p,
                       period, groups, wbyte);
    return hipGetLastError();
}

hipError_t launch_wb(const wb_layout_desc& d, int op, const KArgs& a, hipStream_t stream) {
    const int heads = d.B * d.H;
    const bool small = d.dk == 16;
    switch (d.kind) {
        case WB_FP32:
            return small ? launch_op<WB_FP32, 16, 16>(op, d.mode, a, heads, stream)
                         : launch_op<WB_FP32, 128, 128>(op, d.mode, a, heads, stream);
        case WB_UNIFORM:
            return small ? launch_op<WB_UNIFORM, 16, 16>(op, d.mode, a, heads, stream)
                         : launch_op<WB_UNIFORM, 128, 128>(op, d.mode, a, heads, stream);
        case WB_HAD_INT8:
            if (op == OP_STEP && rot_step_supported(d)) return launch_rot_step(d, a, stream);
            return launch_op<WB_HAD_INT8, 128, 128>(op, d.mode, a, heads, stream);
        case WB_MIXED:
            if (op == OP_STEP && rot_step_supported(d)) return launch_rot_step(d, a, stream);
            return launch_op<WB_MIXED, 128, 128>(op, d.mode, a, heads, stream);
        case WB_HEADALLOC:
            if (op == OP_STEP && headalloc_step_supported(d)) return launch_headalloc_step(d, a, stream);
            return launch_op<WB_BITALLOC, 128, 128>(op, d.mode, a, heads, stream);
        default:
            if (op == OP_STEP && bitalloc_step_supported(d)) return launch_bitalloc_step(d, a, stream);
            return launch_op<WB_BITALLOC, 128, 128>(op, d.mode, a, heads, stream);
    }
}

hipError_t launch_fill(void* dst, size_t n, const uint8_t* pattern, int period, hipStream_t stream) {
    uint4 p{0, 0, 0, 0};
    uint8_t* pb = reinterpret_cast<uint8_t*>(&p);
    for (int i = 0; i < period && i < 16; ++i) pb[i] = pattern[i];
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint8_t*>(dst), n, p, period);
    return hipGetLastError();
}

}  // namespace wb
