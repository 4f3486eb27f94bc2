// Device helpers shared by the write-back kernels (gfx950, wave64).
//
// Pages cited: see include/wbstate.h for the list ([WB], [WB-zh], [LBRS], [LBRS-x],
// [DAMP]).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wbstate.h"

namespace wb {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies with the published constants, the key bumped by the two Weyl constants
// between rounds. Source of the 16-bit uniform draws of stochastic rounding.
struct Ctr4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ Ctr4 philox4x32_10(Ctr4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // each 32 x 32 -> 64-bit product as one multiply (low and high words together)
        const uint64_t p0 = uint64_t(0xD2511F53u) * c.x, p1 = uint64_t(0xCD9E8D57u) * c.z;
        const uint32_t lo0 = uint32_t(p0), hi0 = uint32_t(p0 >> 32);
        const uint32_t lo1 = uint32_t(p1), hi1 = uint32_t(p1 >> 32);
        // (three-input exclusive or: truth table 0x96)
        const uint32_t x0 = uint32_t(__builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96));
        const uint32_t x2 = uint32_t(__builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96));
        c = Ctr4{x0, lo1, x2, lo0};
    }
    return c;
}

// 16-bit draws for the 8 consecutive columns 8*cg .. 8*cg+7 of one stored row.
__device__ __forceinline__ void sr_draws8(uint64_t seed, uint32_t bh, uint64_t t, int row, int cg,
                                          uint32_t r16[8]) {
    const Ctr4 w = philox4x32_10(Ctr4{uint32_t(16 * row + cg), bh, uint32_t(t), uint32_t(t >> 32)},
                                 uint32_t(seed), uint32_t(seed >> 32));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) r16[c] = (c & 1) ? (ws[c >> 1] >> 16) : (ws[c >> 1] & 0xFFFFu);
}

// 16 bytes from global memory straight into LDS (no registers): lane l of the wavefront
// writes bytes [16 l, 16 l + 16) after `wave_dst`, which must be the same for every lane
// of the wavefront (the hardware takes it from a scalar register). The write completes
// with the wavefront's vector-memory counter; the compiler does not order later LDS
// reads after it, so a wavefront that issued such loads calls lds_loads_wait() before
// the workgroup barrier that publishes the data.
__device__ __forceinline__ void lds_load16(const void* src, void* wave_dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)wave_dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_loads_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// float16 conversions. float64 -> float16 must round once, to nearest with ties to
// even: a float64 -> float32 -> float16 chain of two nearest roundings can land on the
// wrong side of a float16 midpoint. The float32 step is therefore rounded to odd
// (truncate, then set the last bit if anything was dropped), which keeps enough
// information for the final nearest rounding to float16 to be the correct rounding of
// the float64 value (Boldo & Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd", IEEE Trans. Computers 57(4), 2008: 24 >=
// 11 + 2 bits). Overflow goes to infinity, values below half the smallest float16
// subnormal to zero.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
    const float f = float(x);
    uint32_t fb = __float_as_uint(f);
    const double back = double(f);
    if (back != x) {
        if (fabs(back) > fabs(x)) fb -= 1u;   // one step toward zero: the truncation
        fb |= 1u;                             // sticky bit: round to odd
    }
    return __half_as_ushort(__float2half_rn(__uint_as_float(fb)));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __half_as_ushort(__float2half_rn(x));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
    return __half2float(__ushort_as_half(uint16_t(bits)));
}

// float16 bits of the product p * q. The bits are made opaque before anything else reads
// them, so that a stored float16 step and the step used for rounding are one value: the
// compiler may fuse the multiply into the conversion (one rounding) or not (two), and
// without the barrier it has been seen to do one for the stored bits and the other for
// the value derived from them.
__device__ __forceinline__ uint32_t f16_bits_of_product(float p, float q) {
    uint32_t b = f32_to_f16_bits(p * q);
    asm volatile("" : "+v"(b));
    return b;
}

template <typename Real>
__device__ __forceinline__ uint16_t to_f16_bits(Real x);
template <>
__device__ __forceinline__ uint16_t to_f16_bits<double>(double x) { return f64_to_f16_bits(x); }
template <>
__device__ __forceinline__ uint16_t to_f16_bits<float>(float x) { return f32_to_f16_bits(x); }

// ---------------------------------------------------------------------------
// Cross-lane helpers (xor butterflies inside a wavefront).
template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// ---------------------------------------------------------------------------
// One write-back rule on the grid offset + kappa * step, kappa in [lo, hi]
// ([WB] / [WB-zh] write-back rules; ties to even and rail clamp per [WB-zh]
// "Reproduction assessment"). Returns kappa; writes the new EF residual.
template <int MODE, typename Real>
__device__ __forceinline__ int round_rule(Real x, Real e, Real step, Real offset, int lo, int hi,
                                          uint32_t r16, float* e_new) {
    if (step == Real(0)) {
        if (MODE == WB_EF) *e_new = 0.f;
        return 0;
    }
    const Real target = (MODE == WB_EF) ? x + e : x;
    const Real tau = (target - offset) / step;
    Real kf;
    if (MODE == WB_SR) {
        const Real fl = floor(tau);
        kf = fl + ((Real(r16) < (tau - fl) * Real(65536)) ? Real(1) : Real(0));
    } else {
        kf = rint(tau);
    }
    kf = fmin(fmax(kf, Real(lo)), Real(hi));
    if (MODE == WB_EF) {
        const Real xhat = offset + kf * step;
        Real r = target - xhat;
        r = fmin(fmax(r, -step), step);
        *e_new = float(r);
    }
    return int(kf);
}

// ---------------------------------------------------------------------------
// Online decay / erasure estimators of one head ([LBRS] "State bit allocation"):
// exponential averages of span 64 (alpha = 2/65 per token) kept unnormalised, as
// [N_a: dk][N_r: dk][W, pad x3] floats: N_a averages 1 - e^{-2 s_i}, N_r averages
// beta (2 - beta) k_i^2, W is the weight sum. One call folds one token into one row
// (and, for row 0, into W).
constexpr float kEmaAlpha = 2.0f / 65.0f, kEmaKeep = 63.0f / 65.0f;
__device__ __forceinline__ int est_stride(int dk) { return 2 * dk + 4; }
__device__ __forceinline__ void ema_fold_row(float* est, int dk, int row, float s, float beta, float k) {
    const float xa = -expm1f(-2.0f * s);
    const float xr = beta * (2.0f - beta) * (k * k);
    est[row] = __builtin_fmaf(est[row], kEmaKeep, kEmaAlpha * xa);
    est[dk + row] = __builtin_fmaf(est[dk + row], kEmaKeep, kEmaAlpha * xr);
    if (row == 0) est[2 * dk] = __builtin_fmaf(est[2 * dk], kEmaKeep, kEmaAlpha);
}

// float64 DPP move inside rows of 16 lanes (both 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

// v + (the value lanes 32 apart / 16 apart hold): the two halves of the wavefront (odd
// and even DPP rows) exchanged by one lane swap per 32-bit half
__device__ __forceinline__ double add_xor32_f64(double v) {
    const uint64_t b = __double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
    return __longlong_as_double((long long)((uint64_t(hi[0]) << 32) | lo[0])) +
           __longlong_as_double((long long)((uint64_t(hi[1]) << 32) | lo[1]));
}
__device__ __forceinline__ double add_xor16_f64(double v) {
    const uint64_t b = __double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
    return __longlong_as_double((long long)((uint64_t(hi[0]) << 32) | lo[0])) +
           __longlong_as_double((long long)((uint64_t(hi[1]) << 32) | lo[1]));
}

// float32 v + the value of the lane 32 / 16 apart (one lane swap)
__device__ __forceinline__ float add_xor32_f32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor16_f32(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over the lanes of the wavefront that are equal modulo NB (1 or 4), returned in
// every lane: DPP inside rows of 16 lanes (xor 1, xor 2; rotations by 8 and 4 combine
// the four lanes of a residue class), then the rows by lane swaps.
template <int NB>
__device__ __forceinline__ double wave_sum_f64(double v) {
    static_assert(NB == 1 || NB == 4, "residue classes of 1 or 4 lanes");
    if constexpr (NB == 1) {
        v += dpp_f64<0xB1>(v);     // xor 1
        v += dpp_f64<0x4E>(v);     // xor 2
    }
    v += dpp_f64<0x128>(v);        // row_ror:8
    v += dpp_f64<0x124>(v);        // row_ror:4
    v = add_xor16_f64(v);
    return add_xor32_f64(v);
}

}  // namespace wb
