// Decode write-back step of the Hadamard-rotated layouts, round to nearest: HAD_INT8
// (every row in the rotated domain, per-block affine INT8) and MIXED (the first k_hi
// physical rows in float16, the rest Hadamard INT8, rows permuted per head).
// [DAMP] "Implementation" (reconstruct, update, re-quantize, write back), "Key
// Points" (transform along the value dimension); [LBRS] "Accumulated readout error".
//
// Same computation as the generic decode kernel (rotated domain: u = sum_P k a S +
// H sum_Q k a Y, w = beta (v - u), S_P' = a S_P + k w, Y_Q' = a Y_Q + k (H w),
// o = sum_P q a S + H sum_Q q a Y + (q . k) w), organised for throughput:
//   * the region is staged in LDS with 16-byte loads, updated there, and written back
//     with 16-byte stores;
//   * u and p (contractions over rows) run column-parallel: thread (j, half) walks
//     half of the rows of column j, so the only cross-thread step is adding two
//     halves; the float64 step and offset of every INT8 block are tabulated once;
//   * the three 128-point transforms run on wavefronts (H uQ then H w on one, H pQ on
//     another);
//   * the update and the requantization run row-parallel (lane = 4 rows x 16 columns,
//     so a block of 32 values spans 2 lanes) with float64 element arithmetic and the
//     block minimum / maximum by DPP;
//   * float64 -> float16 goes through float32 rounded to odd, then the hardware
//     conversion: rounding to odd at 24 bits followed by a rounding to 11 bits gives
//     the correctly rounded result (Boldo & Melquiond, IEEE Trans. Computers 2008).
// Float64 is used wherever a stored code or float16 value is decided: the codes must
// agree with a float64 evaluation to within 1e-5 of a step, and float16 rows to within
// 1e-5 of a float16 spacing.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256;
constexpr double kInvSqrt128 = 0.08838834764831844055;

// IB: bits of the integer tier's codes (8, or 4 with two codes a byte, low nibble first)
template <int KHI, int BLOCK, int IB = 8>
struct RotLayout {
    static constexpr int NQ = DK - KHI;                     // integer rows
    static constexpr int NB = DV / BLOCK;                   // blocks per integer row
    static constexpr int TOP = (1 << IB) - 1;               // largest code
    static constexpr int CODE_BASE = KHI * DV * 2;
    static constexpr int META_BASE = CODE_BASE + NQ * DV * IB / 8;
    static constexpr int REGION = META_BASE + NQ * NB * 4;  // bytes (a multiple of 16)
    static_assert(REGION % 16 == 0, "region must be a whole number of 16-byte words");
};

template <int KHI, int BLOCK, int IB>
struct RotSmem {
    using LY = RotLayout<KHI, BLOCK, IB>;
    // (uP, pP, uQ, pQ) of the second half, then the sums; before the contraction its
    // first half holds (k a, q a) per physical row
    double part[4][DV];
    double2 kqh[KHI > 0 ? KHI : 1];  // (k a, q a) of the float16 rows
    double2 ak[DK];                  // (a, k)
    float2 sz[LY::NQ * LY::NB];      // (step, offset) of every INT8 block (float16 values)
    double2 kqs[LY::NQ * LY::NB];    // (k a step, q a step) of every INT8 block
    double zsum[4][LY::NB][2];       // per wavefront and block column: (sum k a offset, sum q a offset)
    static constexpr int ZW = (LY::NQ * LY::NB + 63) / 64 < 4 ? (LY::NQ * LY::NB + 63) / 64 : 4;
    double w[DV], hw[DV];
    double qk[2];
    uint32_t reg[LY::REGION / 4];
};

__device__ __forceinline__ uint16_t f64_to_f16_rto(double x) {
    const float f = float(x);
    uint32_t fb = __float_as_uint(f);
    const double back = double(f);
    if (back != x) {
        if (fabs(back) > fabs(x)) fb -= 1u;   // one step toward zero: the truncation
        fb |= 1u;                             // sticky bit: round to odd
    }
    return __half_as_ushort(__float2half_rn(__uint_as_float(fb)));
}

__device__ __forceinline__ double f16_to_f64(uint32_t bits) { return double(f16_bits_to_f32(bits)); }

// min and max over the lanes of one block (BLOCK / 16 consecutive lanes of a DPP row)
template <int BLOCK>
__device__ __forceinline__ void block_minmax(double& mn, double& mx) {
    mn = fmin(mn, dpp_f64<0xB1>(mn));     // xor 1
    mx = fmax(mx, dpp_f64<0xB1>(mx));
    if constexpr (BLOCK == 128) {
        mn = fmin(mn, dpp_f64<0x4E>(mn));     // xor 2
        mx = fmax(mx, dpp_f64<0x4E>(mx));
        mn = fmin(mn, dpp_f64<0x141>(mn));    // half mirror (8 lanes)
        mx = fmax(mx, dpp_f64<0x141>(mx));
    }
}

// Butterfly partner at lane ^ D of a float64 value: DPP inside a row of 16 lanes for
// D = 1, 2, 4, 8 (row_ror:n hands lane i the value of lane i - n mod 16), lane swaps of
// the odd and even rows (D = 16) or of the two halves (D = 32): swapping a register with
// itself leaves the even rows' (low half's) values in the first result and the odd
// rows' (high half's) in the second, everywhere.
template <int D>
__device__ __forceinline__ uint32_t xor_partner32(uint32_t b, int lane) {
    if constexpr (D == 1) return uint32_t(__builtin_amdgcn_mov_dpp(int(b), 0xB1, 0xF, 0xF, false));
    if constexpr (D == 2) return uint32_t(__builtin_amdgcn_mov_dpp(int(b), 0x4E, 0xF, 0xF, false));
    if constexpr (D == 4) {
        const int up = __builtin_amdgcn_mov_dpp(int(b), 0x12C, 0xF, 0xF, false);   // lane i + 4
        const int dn = __builtin_amdgcn_mov_dpp(int(b), 0x124, 0xF, 0xF, false);   // lane i - 4
        return uint32_t((lane & 4) ? dn : up);
    }
    if constexpr (D == 8) return uint32_t(__builtin_amdgcn_mov_dpp(int(b), 0x128, 0xF, 0xF, false));
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        return (lane & 16) ? r[0] : r[1];
    }
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return (lane & 32) ? r[0] : r[1];
}

template <int D>
__device__ __forceinline__ double xor_partner(double v, int lane) {
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = xor_partner32<D>(uint32_t(b), lane), hi = xor_partner32<D>(uint32_t(b >> 32), lane);
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

template <int D>
__device__ __forceinline__ void butterfly(double& x, double& y, int lane) {
    const double sg = (lane & D) ? -1.0 : 1.0;    // lane with bit D set: partner - self
    const double ox = xor_partner<D>(x, lane), oy = xor_partner<D>(y, lane);
    x = fma(sg, x, ox);
    y = fma(sg, y, oy);
}

// 128-point orthonormal transform of a vector held by one wavefront (lane l holds
// elements l and l + 64)
__device__ __forceinline__ void wht128(double& a0, double& a1, int lane) {
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

template <int KHI, int BLOCK, int IB>
__global__ void __launch_bounds__(NT) rot_step_kernel(const KArgs A) {
    using LY = RotLayout<KHI, BLOCK, IB>;
    __shared__ RotSmem<KHI, BLOCK, IB> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = blockIdx.x;
    const int h = head % A.H;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    uint8_t* lb = reinterpret_cast<uint8_t*>(sm.reg);
    double2* kq = reinterpret_cast<double2*>(&sm.part[0][0]);
    constexpr int kZW = RotSmem<KHI, BLOCK, IB>::ZW;     // wavefronts that hold INT8 blocks

    // v and beta for the vector phase, requested first
    float v_lo = 0.f, v_hi = 0.f, beta_in = 0.f;
    if (wave == 0) {
        v_lo = A.v[(size_t)head * DV + lane];
        v_hi = A.v[(size_t)head * DV + lane + 64];
        beta_in = A.beta[head];
    }

    // ---- stage the region; per-row tables in physical row order -----------------------
    {
        const uint4* src = reinterpret_cast<const uint4*>(region);
        uint4* dst = reinterpret_cast<uint4*>(sm.reg);
#pragma unroll
        for (int i = tid; i < LY::REGION / 16; i += NT) dst[i] = src[i];
    }
    if (wave < 2) {
        const int p = tid;
        const int lr = KHI > 0 ? int(A.perm[h * DK + p]) : p;
        const double kd = double(A.k[(size_t)head * DK + lr]);
        const double qd = double(A.q[(size_t)head * DK + lr]);
        const float sv = A.s_per_row ? A.s[(size_t)head * DK + lr] : A.s[head];
        const double ad = exp(-double(sv));
        kq[p] = make_double2(kd * ad, qd * ad);
        sm.ak[p] = make_double2(ad, kd);
        double pq = qd * kd;
        pq = wave_sum_f64<1>(pq);
        if (lane == 0) sm.qk[wave] = pq;
    }
    __syncthreads();
    // The contraction over rows folds each INT8 block's step into the row weights:
    // sum_r c_r (offset_rg + code step_rg) = sum_r (c_r step_rg) code + sum_r c_r offset_rg,
    // with the offset sums (one per block column g) formed here once. Thread t handles
    // the blocks t, t + 256, .. (all of block column t % NB).
    {
        double zu = 0.0, zp = 0.0;
        for (int i = tid; i < LY::NQ * LY::NB; i += NT) {
            const uint32_t m = sm.reg[LY::META_BASE / 4 + i];
            const float sc = f16_bits_to_f32(m & 0xFFFFu), zr = f16_bits_to_f32(m >> 16);
            sm.sz[i] = make_float2(sc, zr);
            const double2 c = kq[i / LY::NB + KHI];
            sm.kqs[i] = make_double2(c.x * double(sc), c.y * double(sc));
            zu = fma(c.x, double(zr), zu);
            zp = fma(c.y, double(zr), zp);
        }
        // sum over the lanes of one block column (lanes equal modulo NB), on the
        // wavefronts that hold blocks
        if (wave < kZW) {
            zu = wave_sum_f64<LY::NB>(zu);
            zp = wave_sum_f64<LY::NB>(zp);
            if (lane < LY::NB) {
                sm.zsum[wave][lane][0] = zu;
                sm.zsum[wave][lane][1] = zp;
            }
        }
        if (tid < KHI) sm.kqh[tid] = kq[tid];
    }
    __syncthreads();

    // ---- u, p: thread (j, half) sums half of the rows of column j -----------------------
    {
        const int j = tid & (DV - 1), half = tid >> 7;
        double uP = 0.0, pP = 0.0, uQ = 0.0, pQ = 0.0;
        if constexpr (KHI > 0) {
            const uint16_t* f16rows = reinterpret_cast<const uint16_t*>(lb);
#pragma unroll 4
            for (int p = half * (KHI / 2); p < (half + 1) * (KHI / 2); ++p) {
                const double x = f16_to_f64(f16rows[p * DV + j]);
                const double2 c = sm.kqh[p];
                uP = fma(c.x, x, uP);
                pP = fma(c.y, x, pP);
            }
        }
        const int g = j / BLOCK;
        {
            // two interleaved partial sums per quantity (shorter dependency chains)
            double uQ1 = 0.0, pQ1 = 0.0;
            static_assert(LY::NQ % 4 == 0, "rows are taken two at a time per half");
#pragma unroll 4
            for (int qr = half * (LY::NQ / 2); qr < (half + 1) * (LY::NQ / 2); qr += 2) {
                double code0, code1;
                if constexpr (IB == 8) {
                    code0 = double(lb[LY::CODE_BASE + qr * DV + j]);
                    code1 = double(lb[LY::CODE_BASE + (qr + 1) * DV + j]);
                } else {
                    code0 = double((lb[LY::CODE_BASE + (qr * DV + j) / 2] >> ((j & 1) * 4)) & 15u);
                    code1 = double((lb[LY::CODE_BASE + ((qr + 1) * DV + j) / 2] >> ((j & 1) * 4)) & 15u);
                }
                const double2 c0 = sm.kqs[qr * LY::NB + g];         // (k a step, q a step)
                const double2 c1 = sm.kqs[(qr + 1) * LY::NB + g];
                uQ = fma(c0.x, code0, uQ);
                pQ = fma(c0.y, code0, pQ);
                uQ1 = fma(c1.x, code1, uQ1);
                pQ1 = fma(c1.y, code1, pQ1);
            }
            uQ += uQ1;
            pQ += pQ1;
        }
        if (half == 0) {
#pragma unroll
            for (int wv = 0; wv < kZW; ++wv) {
                uQ += sm.zsum[wv][g][0];
                pQ += sm.zsum[wv][g][1];
            }
        }
        if (half == 1) {
            sm.part[0][j] = uP;
            sm.part[1][j] = pP;
            sm.part[2][j] = uQ;
            sm.part[3][j] = pQ;
        }
        __syncthreads();
        if (half == 0) {
            sm.part[0][j] += uP;
            sm.part[1][j] += pP;
            sm.part[2][j] += uQ;
            sm.part[3][j] += pQ;
        }
        __syncthreads();
    }

    // ---- w = beta (v - u), o = p + (q . k) w, H w (one wavefront) ----------------------
    // (wavefront 0: u, w and H w; wavefront 1: p, in parallel; o after the barrier)
    if (wave == 0) {
        double uq0 = sm.part[2][lane], uq1 = sm.part[2][lane + 64];
        wht128(uq0, uq1, lane);
        const double u0 = sm.part[0][lane] + uq0, u1 = sm.part[0][lane + 64] + uq1;
        const double w0 = double(beta_in) * (double(v_lo) - u0);
        const double w1 = double(beta_in) * (double(v_hi) - u1);
        sm.w[lane] = w0;
        sm.w[lane + 64] = w1;
        double r0 = w0, r1 = w1;
        wht128(r0, r1, lane);
        sm.hw[lane] = r0;
        sm.hw[lane + 64] = r1;
    } else if (wave == 1) {
        double pq0 = sm.part[3][lane], pq1 = sm.part[3][lane + 64];
        wht128(pq0, pq1, lane);
        sm.part[3][lane] = sm.part[1][lane] + pq0;
        sm.part[3][lane + 64] = sm.part[1][lane + 64] + pq1;
    }
    __syncthreads();
    if (tid >= NT - DV) {
        const int j = tid - (NT - DV);
        A.o[(size_t)head * DV + j] = float(sm.part[3][j] + (sm.qk[0] + sm.qk[1]) * sm.w[j]);
    }

    // ---- update and requantize in place (lane = 4 rows x 16 columns) -------------------
    // A block of BLOCK columns of a row spans BLOCK / 16 lanes, so its range, step and
    // offset are derived by few lanes (the per-block work is repeated on each of them).
    {
        const int rg = tid >> 3, cg = tid & 7;
        constexpr int LPB = BLOCK / 16;                     // lanes per block
        double hwv[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) hwv[c] = sm.hw[16 * cg + c];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int p = rg + 32 * m;
            const double2 ak = sm.ak[p];
            if (KHI > 0 && p < KHI) {
                // float16 row (original domain, updated with w itself); the rows below
                // k_hi are those of whole wavefronts at m = 0
                uint4* ptr = reinterpret_cast<uint4*>(lb + (p * DV + 16 * cg) * 2);
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    const uint4 raw = ptr[hv];
                    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
                    uint32_t o4[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const double x = f16_to_f64((w4[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu);
                        const double xn = fma(ak.x, x, ak.y * sm.w[16 * cg + 8 * hv + c]);
                        o4[c >> 1] |= uint32_t(f64_to_f16_rto(xn)) << ((c & 1) * 16);
                    }
                    ptr[hv] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
                }
                continue;
            }
            const int qr = p - KHI;
            const int g = (16 * cg) / BLOCK;
            // the lane's 16 codes: 16 bytes, or 8 bytes of nibbles
            uint8_t* cptr = lb + LY::CODE_BASE + (qr * DV + 16 * cg) * IB / 8;
            uint32_t rw[4];
            if constexpr (IB == 8) {
                const uint4 raw = *reinterpret_cast<const uint4*>(cptr);
                rw[0] = raw.x; rw[1] = raw.y; rw[2] = raw.z; rw[3] = raw.w;
            } else {
                const uint2 raw = *reinterpret_cast<const uint2*>(cptr);
                rw[0] = raw.x; rw[1] = raw.y; rw[2] = 0u; rw[3] = 0u;
            }
            const float2 s = sm.sz[qr * LY::NB + g];
            // a (zero + code * scale) + k (H w)_c = code * (a scale) + (a zero + k (H w)_c)
            const double as = ak.x * double(s.x), az = ak.x * double(s.y);
            double y[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint32_t code = IB == 8 ? (rw[c >> 2] >> ((c & 3) * 8)) & 0xFFu
                                              : (rw[c >> 3] >> ((c & 7) * 4)) & 0xFu;
                y[c] = fma(double(code), as, fma(ak.y, hwv[c], az));
            }
            double mn = y[0], mx = y[0];
#pragma unroll
            for (int c = 1; c < 16; ++c) {
                mn = fmin(mn, y[c]);
                mx = fmax(mx, y[c]);
            }
            block_minmax<BLOCK>(mn, mx);
            // (a product with 1/TOP instead of the quotient: the two differ by at most one
            // float64 unit, which moves a float16 rounding only at a midpoint)
            const uint16_t sbits = f64_to_f16_rto(fmax(mx - mn, 0.0) * (1.0 / double(LY::TOP)));
            const uint16_t zbits = f64_to_f16_rto(mn);
            const double scale = f16_to_f64(sbits), zero = f16_to_f64(zbits);
            uint32_t o4[4] = {0, 0, 0, 0};
            if (scale != 0.0) {
                // reciprocal of the step refined by one Newton step
                double inv = __builtin_amdgcn_rcp(scale);
                inv = fma(fma(-scale, inv, 1.0), inv, inv);
                const double nz = -zero * inv;
                // levels t = (y - zero) / scale lie within +-2^30 unless the offset is far
                // outside the block's range (then the float64 path below is taken)
                const double span = fmax(fabs(mx - zero), fabs(mn - zero)) * inv;
                if (span < 1073741824.0) {
                    // t + 1.5 * 2^52 rounds t to the nearest integer (ties to even); its
                    // low 32 bits are that integer, clamped to [0, TOP] in integer form
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const double r = fma(y[c], inv, nz) + 6755399441055744.0;
                        const int kk = min(max(int(uint32_t(__double_as_longlong(r))), 0), LY::TOP);
                        if constexpr (IB == 8) o4[c >> 2] |= uint32_t(kk) << ((c & 3) * 8);
                        else o4[c >> 3] |= uint32_t(kk) << ((c & 7) * 4);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const double kf = fmin(fmax(rint((y[c] - zero) / scale), 0.0), double(LY::TOP));
                        if constexpr (IB == 8) o4[c >> 2] |= uint32_t(kf) << ((c & 3) * 8);
                        else o4[c >> 3] |= uint32_t(kf) << ((c & 7) * 4);
                    }
                }
            }
            if constexpr (IB == 8) *reinterpret_cast<uint4*>(cptr) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
            else *reinterpret_cast<uint2*>(cptr) = make_uint2(o4[0], o4[1]);
            if ((cg % LPB) == 0)
                sm.reg[LY::META_BASE / 4 + qr * LY::NB + g] = uint32_t(sbits) | (uint32_t(zbits) << 16);
        }
    }
    __syncthreads();
    {
        const uint4* src = reinterpret_cast<const uint4*>(sm.reg);
        uint4* dst = reinterpret_cast<uint4*>(region);
#pragma unroll
        for (int i = tid; i < LY::REGION / 16; i += NT) dst[i] = src[i];
    }
}

template <int KHI, int BLOCK>
hipError_t launch_rot(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.int_bits == 4) hipLaunchKernelGGL((rot_step_kernel<KHI, BLOCK, 4>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((rot_step_kernel<KHI, BLOCK, 8>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool rot_step_supported(const wb_layout_desc& d) {
    if (d.mode != WB_RTN || d.dk != DK || d.dv != DV) return false;
    if (d.kind == WB_HAD_INT8) return d.block == 32 || d.block == 128;
    if (d.kind == WB_MIXED) return d.k_hi == 16 && d.block == 32;
    return false;
}

hipError_t launch_rot_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.kind == WB_MIXED) return launch_rot<16, 32>(d, a, stream);
    return d.block == 32 ? launch_rot<0, 32>(d, a, stream) : launch_rot<0, 128>(d, a, stream);
}

}  // namespace wb
