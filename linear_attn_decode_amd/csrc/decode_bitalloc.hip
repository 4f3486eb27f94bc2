// Decode write-back step for the decay-aware per-row-width layout (BITALLOC), tuned for
// the VALU budget of gfx950.
//
// Same computation as the generic decode kernel (dequantize -> decay -> u = k^T D S ->
// w = beta (v - u) -> S' = D S + k w^T -> o -> Delta_i = f16(f_i R_i / n_i) -> nearest
// level -> pack), organised so that each stored element costs few vector instructions:
//   * rows are visited in order of increasing width, so the 4 rows a wavefront handles
//     per step nearly always share one width; that width is read into a scalar register
//     and the unpack / pack code is chosen by a scalar branch and specialised per width
//     (static bit positions); a group of mixed widths takes a generic per-lane path;
//   * eight wavefronts per head; a lane holds 4 rows x 8 columns of the state (32
//     values as floats, 64 VGPRs: 8 wavefronts per SIMD);
//   * six wavefronts copy the region into LDS with global-to-LDS loads while the other
//     two load the rows' inputs and build the per-row tables, at a raised issue
//     priority (the workgroup waits for them);
//   * the sort, the byte offsets of the rows and their ranks come from wavefront ballots
//     (each of the two wavefronts that build the tables reads the widths of all 128
//     rows, so no cross-wave scan is needed);
//   * per-row constants (decayed step, offset term, k_i, q_i, f_i / n_i, byte offset,
//     width) sit in LDS tables indexed by sorted position;
//   * u and p run on the bfloat16 matrix cores with exact operands (the integer codes,
//     and the row weights split into three bfloat16 limbs); a wavefront's partial sums
//     go to LDS once;
//   * dequantize + decay is one FMA: a_i Delta_i (code - n_i) = code * (a_i Delta_i) +
//     (-n_i a_i Delta_i);
//   * rounding to the nearest level adds 1.5 * 2^23 in the same FMA as the scaling
//     (x * (1/Delta) + magic rounds the exact product once, ties to the even level),
//     clamps with one med3 to [magic - n_i, magic + n_i], and packs with shift-adds whose
//     constant high bits (those of magic - n_i, so the field is level + n_i) are removed
//     once per 32-bit word;
//   * row maxima use DPP integer max on the bits of |x| (ordered like the values);
//   * the packed codes of a lane (8 elements = b bytes) and each row's new Delta go
//     straight to the region in HBM at their final byte offsets (a decode step changes
//     no width, so rows keep their offsets), with no staging copy or final barrier.
// Two more instantiations widen it: the layer-wise budget (the code area holds every
// row at b_max; the widths are read first and only the codes in use are staged and
// stored, so the zero tail is never touched) and one-bit rows (the two levels
// -Delta, +Delta: the code is the sign, Delta = f16(mean |x|) from a row sum).
// Layout citations: [LBRS] "State bit allocation", "Levels and storage".
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128;
constexpr int NW = 8, NT = 64 * NW;            // wavefronts per head
constexpr int NG = 4 * NW;                     // row groups: a wavefront step covers 4 rows
constexpr int MR = DK / NG;                    // rows per lane
constexpr float kMagic = 12582912.0f;          // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

struct TabA {                                   // dequantize constants, by sorted position
    float alpha, beta0, k, q;                   // a Delta, -n a Delta, k_i, q_i
};
struct TabB {                                   // requantize constants, by sorted position
    uint32_t off;                               // byte offset of the row's codes
    uint32_t bw;                                // width (off, bw: one 8-byte read)
    float fn;                                   // f / n
    uint32_t row;                               // row index
};

struct BaFixed {
    TabA ta[DK];
    TabB tb[DK];
    float red[2][NW][DV];                      // u / p partials of the wavefronts
    float w[DV];
    float qk[4];
    float bias[2][2];                          // per table wavefront: sum k beta0, sum q beta0
    // bfloat16 limbs of the matrix-core row weights k_i alpha_i and q_i alpha_i, by
    // [wavefront][row group][row step][quantity * 4 + limb] (limb 3 is zero)
    uint16_t alimb[NW][4][MR][8];
};
// LDS: the staged region first (at most the code area at 8 bits per element, Delta and
// the width / fit bytes, and 16 bytes that the last row's 3-word read may touch), then
// BaFixed; one static size, so that the compiler folds the bases into the instruction
// offsets
constexpr int kCodeAreaMax = DK * DV;
constexpr int kFixedOffset = (kCodeAreaMax + 3 * DK + 16 + 15) / 16 * 16;
constexpr int kSmemBytes = kFixedOffset + int(sizeof(BaFixed));

// f_k / n_b for fit index k (f_k = 1/4 + k/20) and width b (n_b = 2^(b-1) - 1), each
// step rounded once in float32 (the multiply and add kept apart, the division correctly
// rounded); computed in registers, so that no memory lookup sits on the table path.
// One-bit rows (b = 1, no fit) get 0.
__device__ __forceinline__ float fn_of(int k, int b) {
    const float f = __fadd_rn(0.25f, __fmul_rn(0.05f, float(k)));
    return b > 1 ? __fdiv_rn(f, float((1 << (b - 1)) - 1)) : 0.f;
}

// The three 32-bit words of the staged region that hold a lane's 8 codes (at most 64
// bits starting anywhere in the first word).
struct Raw {
    uint32_t w0, w1, w2;
};
__device__ __forceinline__ Raw load_raw(const uint32_t* reg, int boff) {
    const int wi = boff >> 2;
    return Raw{reg[wi], reg[wi + 1], reg[wi + 2]};
}

// 0x0F0F0F0F mask kept opaque, so the byte conversions below stay byte conversions
__device__ __forceinline__ uint32_t low_nibbles(uint32_t v) {
    uint32_t r;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(r) : "v"(v));
    return r;
}

// 8 codes of `B` bits starting at bit 8 * (boff & 3) of the raw words.
template <int B>
__device__ __forceinline__ void unpack8(const Raw& raw, int boff, float code[8]) {
    if constexpr (B == 4) {                            // 4-byte aligned
        const uint32_t lo = low_nibbles(raw.w0), hi = low_nibbles(raw.w0 >> 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            code[2 * c] = float((lo >> (8 * c)) & 255u);
            code[2 * c + 1] = float((hi >> (8 * c)) & 255u);
        }
    } else if constexpr (B == 8) {                     // 8-byte aligned
#pragma unroll
        for (int c = 0; c < 4; ++c) code[c] = float((raw.w0 >> (8 * c)) & 255u);
#pragma unroll
        for (int c = 0; c < 4; ++c) code[4 + c] = float((raw.w1 >> (8 * c)) & 255u);
    } else {
        const int sh = (boff & 3) * 8;
        const uint32_t lo = __builtin_amdgcn_alignbit(raw.w1, raw.w0, sh);
        const uint32_t hi = __builtin_amdgcn_alignbit(raw.w2, raw.w1, sh);
        constexpr uint32_t M = (1u << B) - 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int p = c * B;
            uint32_t v;
            if (p + B <= 32) v = (lo >> p) & M;
            else if (p >= 32) v = (hi >> (p - 32)) & M;
            else v = __builtin_amdgcn_alignbit(hi, lo, p) & M;
            code[c] = float(v);
        }
    }
}

// (y << s) + a as one instruction (the compiler otherwise splits such chains into
// shifts and three-input adds)
__device__ __forceinline__ uint32_t lshl_add(uint32_t y, int s, uint32_t a) {
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(y), "i"(s), "v"(a));
    return r;
}

// 1 / Delta of the 8 values of a lane: one per row (InvOne) or one per column (InvCol)
struct InvOne {
    float v;
    __device__ __forceinline__ float operator[](int) const { return v; }
};
struct InvCol {
    const float* p;
    __device__ __forceinline__ float operator[](int c) const { return p[c]; }
};

// Write 8 codes of `B` bits, given in magic-number form (the bits of 1.5 * 2^23 + level,
// level in [-n, n]; the stored field is level + n, n = 2^(B-1) - 1, and 0 / 1 for B = 1),
// or, with FIELD, as the stored fields themselves, packed at byte `boff` of `reg` (B bytes;
// the region in HBM, or a staging copy in LDS).
template <int B, bool FIELD = false>
__device__ __forceinline__ void store8(uint32_t* reg, int boff_i, const uint32_t y[8]) {
    const uint32_t boff = uint32_t(boff_i);     // (unsigned: a scalar base plus a 32-bit lane offset)
    // bits of 1.5 * 2^23 - n: subtracting them leaves level + n
    constexpr uint32_t base = FIELD ? 0u : kMagicBits - uint32_t(B == 1 ? 0 : (1 << (B - 1)) - 1);
    if constexpr (B == 1) {
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) w |= (y[c] - base) << c;
        reinterpret_cast<uint8_t*>(reg)[boff] = uint8_t(w);
        return;
    }
    // the constant high bits of every shifted y are removed once per word
    uint32_t g0 = 0, g1 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int p = c * B;
        if (p + B <= 32) g0 += base << p;
        else if (p >= 32) g1 += base << (p - 32);
    }
    uint32_t w0 = y[0] - g0, w1 = 0u - g1;
    bool w1_started = false;
#pragma unroll
    for (int c = 1; c < 8; ++c) {
        const int p = c * B;
        if (p + B <= 32) {
            w0 = lshl_add(y[c], p, w0);
        } else if (p >= 32) {
            if (!w1_started && p == 32) w1 = y[c] + w1;
            else w1 = lshl_add(y[c], p - 32, w1);
            w1_started = true;
        } else {
            const uint32_t code = y[c] - base;
            w0 = lshl_add(code, p, w0);
            w1 += code >> (32 - p);
            w1_started = true;
        }
    }
    uint8_t* bytes = reinterpret_cast<uint8_t*>(reg);
    if constexpr (B == 2) {
        *reinterpret_cast<uint16_t*>(bytes + boff) = uint16_t(w0);
    } else if constexpr (B == 4) {
        *reinterpret_cast<uint32_t*>(bytes + boff) = w0;
    } else if constexpr (B == 8) {
        *reinterpret_cast<uint2*>(bytes + boff) = make_uint2(w0, w1);
    } else if constexpr (B == 6) {
        uint16_t* hw = reinterpret_cast<uint16_t*>(bytes + boff);   // 2-byte aligned
        hw[0] = uint16_t(w0);
        hw[1] = uint16_t(w0 >> 16);
        hw[2] = uint16_t(w1);
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i) (bytes + boff)[i] = uint8_t(i < 4 ? (w0 >> (8 * i)) : (w1 >> (8 * (i - 4))));
    }
}

// Round 8 values to the nearest level (magic-number FMA, med3 clamp) and store them.
template <int B, typename Inv = InvOne>
__device__ __forceinline__ void pack8(uint32_t* reg, int boff, const float x[8], Inv inv) {
    uint32_t y[8];
    if constexpr (B == 1) {
        // one-bit row, round to nearest on -Delta + k 2 Delta: k = 1 exactly where x > 0
        // (an exact zero is the tie, which goes to the even index 0; a zero step stores 0)
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] = kMagicBits + uint32_t(x[c] * inv[c] > 0.f);
    } else {
        // the level itself is rounded (ties to even), then clamped to [-n, n]
        constexpr float n = float((1 << (B - 1)) - 1);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            y[c] = __float_as_uint(
                __builtin_amdgcn_fmed3f(__builtin_fmaf(x[c], inv[c], kMagic), kMagic - n, kMagic + n));
    }
    store8<B>(reg, boff, y);
}

// Stochastic rounding of one value on the grid of the row (level index in [0, 2n], or
// [0, 1] for a one-bit row on -Delta + k 2 Delta): floor(tau) + [u < frac(tau)] with u the
// 16-bit draw over 2^16, clamped at the rails; a zero step stores level 0. Returned in
// magic-number form, 1.5 * 2^23 + level (level in [-n, n], or k for a one-bit row).
__device__ __forceinline__ uint32_t sr_level(float x, float inv, int bw, uint32_t r16) {
    const bool one = bw == 1;
    const float n = one ? 0.f : float((1 << (bw - 1)) - 1);
    const float tau = one ? (inv > 0.f ? __builtin_fmaf(x, 0.5f * inv, 0.5f) : 0.f) : x * inv;
    const float fl = floorf(tau);
    float k = fl + ((float(r16) < (tau - fl) * 65536.f) ? 1.f : 0.f);
    k = one ? __builtin_amdgcn_fmed3f(k, 0.f, 1.f) : __builtin_amdgcn_fmed3f(k, -n, n);
    return __float_as_uint(kMagic + k);
}

// The same rounding for B >= 2 bits in integer form, returning the stored field level + n.
// With tau = x / Delta, F = floor(tau) and g = frac(tau) 2^16, a 16-bit integer draw u has
// u < g exactly when u < ceil(g), so floor(tau) + [u < g] = F + [ceil(g) + 2^16 - 1 - u >=
// 2^16], which is floor((ceil(tau 2^16) + 2^16 - 1 - u) / 2^16) because ceil(tau 2^16) =
// F 2^16 + ceil(g). tau 2^16 is the rounded product scaled by a power of two (exact), its
// ceiling is minus one floor conversion of x * (-2^16 / Delta) (`ninv16`), and the field
// comes out of one arithmetic shift, n 2^16 added before it, clamped to [0, 2n]. A zero
// step (ninv16 = 0) gives the field n, level 0.
__device__ __forceinline__ int cvt_floor_i32(float v) {
    int r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ uint32_t sr_field_int(float x, float ninv16, int n, uint32_t r16) {
    const int z = cvt_floor_i32(x * ninv16);                     // -ceil(tau 2^16)
    const int l = ((n << 16) + 65535 - z - int(r16)) >> 16;      // level + n
    return uint32_t(min(max(l, 0), 2 * n));
}
// Either form for one element of a B-bit row (B = 1: the one-bit grid of sr_level).
template <int B>
__device__ __forceinline__ uint32_t sr_field(float x, float inv, float ninv16, uint32_t r16) {
    if constexpr (B == 1) return sr_level(x, inv, 1, r16) - kMagicBits;
    else return sr_field_int(x, ninv16, (1 << (B - 1)) - 1, r16);
}

template <int B>
__device__ __forceinline__ void pack8_sr(uint32_t* reg, int boff, const float x[8], float inv, const uint32_t r16[8]) {
    const float ninv16 = inv * -65536.f;
    uint32_t y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = sr_field<B>(x[c], inv, ninv16, r16[c]);
    store8<B, true>(reg, boff, y);
}

// Generic unpack / pack for a per-lane width (a group of rows of mixed widths).
__device__ __forceinline__ void unpack8_any(const Raw& raw, int boff, int bw, float code[8]) {
    const int sh = (boff & 3) * 8;
    const uint32_t lo = __builtin_amdgcn_alignbit(raw.w1, raw.w0, sh);
    const uint32_t hi = __builtin_amdgcn_alignbit(raw.w2, raw.w1, sh);
    const uint64_t fld = uint64_t(lo) | (uint64_t(hi) << 32);
    const uint32_t mask = (1u << bw) - 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) code[c] = float(uint32_t(fld >> __umul24(uint32_t(c), uint32_t(bw))) & mask);
}

template <bool OB, bool SR>
__device__ __forceinline__ void pack8_any(uint32_t* reg, int boff, int bw, const float x[8], float inv,
                                          const uint32_t r16[8]) {
    const int ni = (OB && bw == 1) ? 0 : (1 << (bw - 1)) - 1;
    const float n = float(ni);
    const uint32_t base = kMagicBits - uint32_t(ni);     // the field is level + n
    uint64_t fld = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t code;
        if constexpr (SR) {
            code = (OB && bw == 1) ? sr_level(x[c], inv, 1, r16[c]) - kMagicBits
                                   : sr_field_int(x[c], inv * -65536.f, ni, r16[c]);
        } else {
            const uint32_t y = __float_as_uint(
                __builtin_amdgcn_fmed3f(__builtin_fmaf(x[c], inv, kMagic), kMagic - n, kMagic + n));
            code = y - base;
            if (OB && bw == 1) code = x[c] * inv > 0.f;
        }
        fld |= uint64_t(code) << __umul24(uint32_t(c), uint32_t(bw));
    }
    uint8_t* bytes = reinterpret_cast<uint8_t*>(reg) + uint32_t(boff);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < bw) bytes[i] = uint8_t(fld >> (8 * i));
}

// Unpack / pack with the width held per lane. When the lanes share one width (rows
// handled together are adjacent in the width order, so this is the common case), the
// width is a scalar and the specialised code is chosen by a scalar branch; otherwise
// the generic per-lane code runs.
// The floats are pinned inside each specialised branch (an empty asm that takes them as
// operands), so the conversions stay next to the width-specific field extraction (byte
// conversions for widths 4 and 8) instead of being merged after the branches.
template <int B>
__device__ __forceinline__ void unpack8_pinned(const Raw& raw, int boff, float code[8]) {
    unpack8<B>(raw, boff, code);
    asm volatile("" : "+v"(code[0]), "+v"(code[1]), "+v"(code[2]), "+v"(code[3]), "+v"(code[4]), "+v"(code[5]),
                 "+v"(code[6]), "+v"(code[7]));
}

// Returns the width as a scalar when the lanes share it, else 0 (the pack reuses it).
template <bool OB>
__device__ __forceinline__ int unpack_rows(const Raw& raw, int boff, int bw, float code[8]) {
    const int bu = __builtin_amdgcn_readfirstlane(bw);
    if (__ballot(bw != bu) == 0ull) {
        if (OB && bu == 1) {
            unpack8_pinned<1>(raw, boff, code);
            return bu;
        }
        switch (bu) {
            case 2: unpack8_pinned<2>(raw, boff, code); break;
            case 3: unpack8_pinned<3>(raw, boff, code); break;
            case 4: unpack8_pinned<4>(raw, boff, code); break;
            case 5: unpack8_pinned<5>(raw, boff, code); break;
            case 6: unpack8_pinned<6>(raw, boff, code); break;
            case 7: unpack8_pinned<7>(raw, boff, code); break;
            default: unpack8_pinned<8>(raw, boff, code); break;
        }
        return bu;
    }
    unpack8_any(raw, boff, bw, code);
    return 0;
}

template <int B, bool SR>
__device__ __forceinline__ void pack8_rule(uint32_t* reg, int boff, const float x[8], float inv, const uint32_t r16[8]) {
    if constexpr (SR) pack8_sr<B>(reg, boff, x, inv, r16);
    else pack8<B>(reg, boff, x, InvOne{inv});
}

// bu: the shared width from unpack_rows (0: the lanes' widths differ; the per-lane
// width is then read from *bw)
template <bool OB, bool SR>
__device__ __forceinline__ void pack_rows(uint32_t* reg, int boff, int bu, const uint32_t* bw, const float x[8],
                                          float inv, const uint32_t r16[8]) {
    if (bu != 0) {
        if (OB && bu == 1) {
            pack8_rule<1, SR>(reg, boff, x, inv, r16);
            return;
        }
        switch (bu) {
            case 2: pack8_rule<2, SR>(reg, boff, x, inv, r16); break;
            case 3: pack8_rule<3, SR>(reg, boff, x, inv, r16); break;
            case 4: pack8_rule<4, SR>(reg, boff, x, inv, r16); break;
            case 5: pack8_rule<5, SR>(reg, boff, x, inv, r16); break;
            case 6: pack8_rule<6, SR>(reg, boff, x, inv, r16); break;
            case 7: pack8_rule<7, SR>(reg, boff, x, inv, r16); break;
            default: pack8_rule<8, SR>(reg, boff, x, inv, r16); break;
        }
    } else {
        pack8_any<OB, SR>(reg, boff, int(*bw), x, inv, r16);
    }
}

// sum over the wavefront, returned as a scalar (DPP inside rows of 16 lanes, then the
// four row sums)
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// float sum over the wavefront, left in lane 63: DPP inside rows of 16 lanes, then
// each row's sum carried into the next by row broadcasts (lane 15 of row r to row r + 1,
// lane 31 to rows 2 and 3)
__device__ __forceinline__ float wave_sum_f32_last(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// Three bfloat16 limbs whose sum is the float32 c exactly: each limb keeps the leading
// 8 significant bits of what the previous ones left (truncation), and 3 x 8 bits cover
// the 24-bit significand. Returned as (limb0 | limb1 << 16, limb2).
__device__ __forceinline__ uint2 bf16_limbs3(float c) {
    const uint32_t h0 = __float_as_uint(c) & 0xFFFF0000u;
    const float r1 = c - __uint_as_float(h0);
    const uint32_t h1 = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(h1);
    return make_uint2((h0 >> 16) | h1, __float_as_uint(r2) >> 16);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D = A B on the matrix cores (16 x 16 output, K = 32, bfloat16 operands, float32
// accumulation); the operands are four 32-bit registers of two bfloat16 each
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(const uint32_t a[4], const uint32_t b[4]) {
    const uint4 av = make_uint4(a[0], a[1], a[2], a[3]), bv = make_uint4(b[0], b[1], b[2], b[3]);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// DPP moves inside rows of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

// Error feedback on a row of step `dl` (1 / dl = `inv`): y + e rounded to the nearest level
// (magic-number form, as pack8), x-hat = level * dl, and the new residual
// clip(y + e - x-hat, -step, step) left in e. A one-bit row's levels are -dl, +dl (step
// 2 dl: the level is 1 exactly where y + e > 0). A zero step gives level 0 and residual 0.
template <bool OB>
__device__ __forceinline__ void ef_round8(const float x[8], float e[8], float inv, float dl, int bw, uint32_t y[8]) {
    if (OB && bw == 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float t = x[c] + e[c];
            const bool k = t * inv > 0.f;
            y[c] = kMagicBits + uint32_t(k);
            e[c] = fminf(fmaxf(t - (k ? dl : -dl), -2.f * dl), 2.f * dl);
        }
    } else {
        const float n = float((1 << (bw - 1)) - 1);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float t = x[c] + e[c];
            const float yf = __builtin_amdgcn_fmed3f(__builtin_fmaf(t, inv, kMagic), kMagic - n, kMagic + n);
            y[c] = __float_as_uint(yf);
            e[c] = fminf(fmaxf(t - (yf - kMagic) * dl, -dl), dl);
        }
    }
}

// Pack 8 levels in magic-number form at the row's width: specialised when the lanes share
// it (bu, a scalar), else per lane (bw).
template <bool OB>
__device__ __forceinline__ void store_rows(uint32_t* reg, int boff, int bu, int bw, const uint32_t y[8]) {
    if (bu != 0) {
        if (OB && bu == 1) {
            store8<1>(reg, boff, y);
            return;
        }
        switch (bu) {
            case 2: store8<2>(reg, boff, y); break;
            case 3: store8<3>(reg, boff, y); break;
            case 4: store8<4>(reg, boff, y); break;
            case 5: store8<5>(reg, boff, y); break;
            case 6: store8<6>(reg, boff, y); break;
            case 7: store8<7>(reg, boff, y); break;
            default: store8<8>(reg, boff, y); break;
        }
        return;
    }
    const uint32_t base = kMagicBits - uint32_t((OB && bw == 1) ? 0 : (1 << (bw - 1)) - 1);
    uint64_t fld = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) fld |= uint64_t(y[c] - base) << __umul24(uint32_t(c), uint32_t(bw));
    uint8_t* bytes = reinterpret_cast<uint8_t*>(reg) + uint32_t(boff);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < bw) bytes[i] = uint8_t(fld >> (8 * i));
}

// Row maxima (non-negative floats as bit patterns) of the 4 rows a lane holds, reduced
// over the 16 lanes of its DPP row and scattered: lane cg ends with the maximum of row
// ((cg & 1) << 1) | ((cg >> 1) & 1), the four rows spread over every quad.
__device__ __forceinline__ uint32_t rowmax4_scatter(const uint32_t m[4], int cg) {
    const bool odd = cg & 1, hi = cg & 2;
    const uint32_t k0 = odd ? m[2] : m[0], k1 = odd ? m[3] : m[1];
    const uint32_t s0 = odd ? m[0] : m[2], s1 = odd ? m[1] : m[3];
    const uint32_t n0 = max(k0, dpp_u32<0xB1>(s0)), n1 = max(k1, dpp_u32<0xB1>(s1));   // xor 1
    uint32_t v = max(hi ? n1 : n0, dpp_u32<0x4E>(hi ? n0 : n1));                         // xor 2
    v = max(v, dpp_u32<0x124>(v));                                                      // row_ror:4
    return max(v, dpp_u32<0x128>(v));                                                   // row_ror:8
}
// the same for sums of floats
__device__ __forceinline__ float rowsum4_scatter(const float m[4], int cg) {
    const bool odd = cg & 1, hi = cg & 2;
    const float k0 = odd ? m[2] : m[0], k1 = odd ? m[3] : m[1];
    const float s0 = odd ? m[0] : m[2], s1 = odd ? m[1] : m[3];
    const float n0 = k0 + __uint_as_float(dpp_u32<0xB1>(__float_as_uint(s0)));
    const float n1 = k1 + __uint_as_float(dpp_u32<0xB1>(__float_as_uint(s1)));
    float v = (hi ? n1 : n0) + __uint_as_float(dpp_u32<0x4E>(__float_as_uint(hi ? n0 : n1)));
    v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
    return v + __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
}

// EST: fold the token into the attached online estimators; LAYER: the layer-wise budget
// layout (code area of b_max bits per element, codes in use first, then a zero tail);
// OB: one-bit rows may occur; RULE: round to nearest, stochastic rounding with the
// Philox draws of the element (row, 8 columns), or error feedback with the element's
// float32 residual (physical rows, read and written at the row's rounding). Each is its
// own instantiation, so that the plain step carries no trace of the others.
template <bool EST, bool LAYER, bool OB, int RULE>
__global__ void __launch_bounds__(NT, RULE == WB_RTN ? 8 : 6) bitalloc_step_kernel(const KArgs A) {
    constexpr bool SR = RULE == WB_SR, EF = RULE == WB_EF;
    __shared__ __align__(16) uint8_t smraw[kSmemBytes];
    BaFixed& sm = *reinterpret_cast<BaFixed*>(smraw + kFixedOffset);
    uint32_t* reg = reinterpret_cast<uint32_t*>(smraw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = blockIdx.x;
    const int cg = lane & 15, rq = lane >> 4;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    // the code area: the head's codes (per-head budget), or room for every row at b_max
    // with the codes in use first (layer budget); Delta and the width / fit bytes follow
    const int code_bytes = LAYER ? A.code_cap : DK * DV * A.bbar / 8;
    constexpr int kMetaVec = 3 * DK / 16;
    const uint8_t* meta = region + code_bytes + 2 * DK;

    // ---- loads: per-row inputs, the region (straight into LDS) ------------------------
    // Wavefronts 0 and 1 build the per-row tables: they load the rows' inputs only, so
    // that their wait covers nothing else. Wavefronts 2..7 copy the region: per-head
    // budget, the region in one piece; layer budget, the codes every head holds (b_min
    // bits per element) and the metadata, then, once the widths are summed, the rest of
    // the codes in use. Vector i of the region goes to vector i of the staging copy.
    const float vj = A.v[(size_t)head * DV + (tid & (DV - 1))];
    const float beta = A.beta[head];
    const int trow = lane + 64 * (wave & 1);
    const size_t rb = (size_t)head * DK + trow;
    int meta0 = 0, meta1 = 0;
    float kr = 0.f, qr = 0.f, sr = 0.f;
    uint32_t dold = 0;
    int ncode = 0;
    if (LAYER || wave < 2) {
        meta0 = meta[lane];
        meta1 = meta[lane + 64];
    }
    // layer budget: the 16-byte vectors of codes in use, the sum of the widths times
    // DV / 128 (at most the code area)
    if constexpr (LAYER) ncode = min(wave_sum_i32((meta0 & 7) + (meta1 & 7) + 2) * (DV / 128), code_bytes / 16);
    if (wave < 2) {
        kr = A.k[rb];
        qr = A.q[rb];
        sr = A.s_per_row ? A.s[rb] : A.s[head];
        dold = reinterpret_cast<const uint16_t*>(region + code_bytes)[trow];
    } else {
        const uint4* src = reinterpret_cast<const uint4*>(region);
        constexpr int NS = NT - 128;                    // copying threads
        const int st = tid - 128, sw0 = 64 * (wave - 2);
        // vectors [v0, v1): thread st copies v0 + st, v0 + st + NS, ...; the wavefront's
        // first vector of each round is a scalar (the LDS destination comes from it)
        auto copy = [&](int v0, int v1) {
            for (int r = 0; v0 + r + st < v1; r += NS) lds_load16(src + v0 + r + st, reg + 4 * (v0 + r + sw0));
        };
        if constexpr (!LAYER) {
            copy(0, (code_bytes + 3 * DK) / 16);
        } else {
            const int nmin = A.bmin * (DK * DV / 8 / 16);
            copy(0, nmin);
            copy(code_bytes / 16, code_bytes / 16 + kMetaVec);
            copy(nmin, ncode);
        }
        lds_loads_wait();
    }

    // ---- per-row tables: wavefronts 0 and 1 own rows lane and lane + 64 ---------------
    // The width order, the byte offsets and the ranks come from ballots over the width
    // bytes of all 128 rows, which both wavefronts read.
    if (wave < 2) {
        // The rest of the workgroup waits for these two wavefronts: they run at a raised
        // issue priority until the tables are written (other workgroups on the compute
        // unit fill the gaps).
        __builtin_amdgcn_s_setprio(3);
        // (opaque from here on, so that no use of the row inputs is placed among the loads
        // and makes the wavefront wait for them before the loads are all issued)
        asm volatile("" : "+v"(meta0), "+v"(meta1), "+v"(kr), "+v"(qr), "+v"(sr), "+v"(dold));
        if constexpr (EST) ema_fold_row(A.est + (size_t)head * est_stride(DK), DK, trow, sr, beta, kr);
        const int bw0 = (meta0 & 7) + 1, bw1 = (meta1 & 7) + 1;
        const bool hi_half = wave == 1;
        const int bwt = hi_half ? bw1 : bw0;
        int off = 0, pos = 0, before = 0, sum_lo = 0;
#pragma unroll
        for (int v = OB ? 1 : 2; v <= 8; ++v) {
            const unsigned long long ma = __ballot(bw0 == v), mb = __ballot(bw1 == v);
            const int ca = __popcll(ma), cb = __popcll(mb);
            const int bt = lanes_below(hi_half ? mb : ma);
            off += v * bt;
            if (bwt == v) pos = before + (hi_half ? ca : 0) + bt;
            before += ca + cb;
            sum_lo += v * ca;
        }
        if (hi_half) off += sum_lo;
        const int fit = (hi_half ? meta1 : meta0) >> 4;
        const float n = float((1 << (bwt - 1)) - 1);
        const float ad = expf(-sr) * f16_bits_to_f32(dold);
        // dequantize + decay: x = code * alpha + beta0 (a one-bit row's levels are -Delta,
        // +Delta: code * 2 a Delta - a Delta)
        const bool one = OB && bwt == 1;
        const float alpha = one ? 2.f * ad : ad, beta0 = one ? -ad : -n * ad;
        sm.ta[pos] = TabA{alpha, beta0, kr, qr};
        sm.tb[pos] = TabB{uint32_t(off * (DV / 8)), uint32_t(bwt), fn_of(fit, bwt), uint32_t(trow)};
        // u and p on the matrix cores: u_j = sum_i (k_i alpha_i) code_ij + sum_i k_i beta0_i
        // (p with q_i); the row weights as exact bfloat16 limbs, the constant terms summed here
        const uint2 lu = bf16_limbs3(kr * alpha), lp = bf16_limbs3(qr * alpha);
        *reinterpret_cast<uint4*>(&sm.alimb[(pos % NG) >> 2][pos & 3][pos / NG][0]) =
            make_uint4(lu.x, lu.y, lp.x, lp.y);
        // q . k and the constant terms over the wavefront's 64 rows
        const float qsum = wave_sum_f32_last(qr * kr);
        const float bu = wave_sum_f32_last(kr * beta0), bp = wave_sum_f32_last(qr * beta0);
        if (lane == 63) {
            sm.qk[wave] = qsum;
            sm.bias[wave][0] = bu;
            sm.bias[wave][1] = bp;
        }
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();

    // ---- dequantize the lane's 4 rows x 8 columns; u, p on the matrix cores -----------
    // The code words of row m + 1 are requested (and the location of row m + 2 read)
    // before row m is unpacked, so their LDS latency overlaps the arithmetic.
    // Matrix-core operands (16 x 16 x 32, bfloat16): the K slots of lane group rq are the
    // lane's rows m = 0..3 times the two columns of a column pair; B for column pair cp
    // holds the codes (exact in bfloat16), A the limbs of the row weights; output row
    // 8 s + 4 q + limb of lane column cg is the partial of quantity q (u, p) for column
    // 8 cg + 2 cp + s over the wavefront's 16 rows.
    // (byte offset, width) of the lane's row at step m; the lane's codes start at
    // offset + cg * width
    // the wavefront's table entries: sorted positions NG m + 4 wave + rq
    const TabA* taw = &sm.ta[4 * wave];
    const TabB* tbw = &sm.tb[4 * wave];
    auto loc_of = [&](int m) { return *reinterpret_cast<const uint2*>(&tbw[NG * m + rq].off); };
    auto boff_of = [&](uint2 l) { return int(__umul24(uint32_t(cg), l.y) + l.x); };
    // the codes as floats, row m column 8 cg + c; later the updated state in place
    float x[MR][8];
    int bus[MR];                                // shared widths, kept for the pack
    uint2 loc_cur = loc_of(0);
    uint2 loc_next = loc_of(1);
    Raw raw_next = load_raw(reg, boff_of(loc_cur));
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const Raw raw = raw_next;
        const uint2 loc = loc_cur;
        if (m + 1 < MR) {
            raw_next = load_raw(reg, boff_of(loc_next));
            loc_cur = loc_next;
        }
        if (m + 2 < MR) loc_next = loc_of(m + 2);
        bus[m] = unpack_rows<OB>(raw, boff_of(loc), int(loc.y), x[m]);
    }
    {
        // A operand of lane (g = rq, output row mo = cg): the limb of quantity (mo / 4) % 2
        // for each row m in the slot of column parity mo / 8 (limb 3 reads a zero)
        const int mo = cg;
        const uint16_t* al = &sm.alimb[wave][rq][0][((mo >> 2) & 1) * 4 + (mo & 3)];
        uint32_t aop[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) aop[m] = uint32_t(al[8 * m]) << (16 * (mo >> 3));
        // lane (rq, cg) receives quantity rq % 2 of column 8 cg + 2 cp + rq / 2
        float* red = &sm.red[rq & 1][wave][8 * cg + (rq >> 1)];
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) {
            // the codes are integers below 2^8, so a float's high half is its exact bfloat16
            uint32_t bop[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m)
                bop[m] = __builtin_amdgcn_perm(__float_as_uint(x[m][2 * cp + 1]), __float_as_uint(x[m][2 * cp]),
                                               0x07060302u);
            const f32x4_t d = mfma_bf16_16x16x32(aop, bop);
            red[2 * cp] = (d[0] + d[1]) + d[2];
        }
    }
    __syncthreads();

    // ---- w = beta (v - u) (threads 0..127); p summed by threads 128..255 for o --------
    const int jq = tid >> 7, j = tid & (DV - 1);
    float pj = 0.f;
    if (jq < 2) {
        float acc = sm.bias[0][jq] + sm.bias[1][jq];
#pragma unroll
        for (int g = 0; g < NW; ++g) acc += sm.red[jq][g][j];
        if (jq == 0) sm.w[j] = beta * (vj - acc);
        else pj = acc;
    }
    __syncthreads();
    if (jq == 1) {
        const float qk = sm.qk[0] + sm.qk[1];
        A.o[(size_t)head * DV + j] = __builtin_fmaf(qk, sm.w[j], pj);
    }

    // ---- update, requantize and store ---------------------------------------------------
    float wv[8];
    {
        const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[8 * cg]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[8 * cg + 4]);
        wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
        wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
    }
    // the new codes and steps go straight to the region in HBM (the rows keep their
    // offsets: a decode step changes no width), each lane storing what it rounded
    uint32_t* gout = reinterpret_cast<uint32_t*>(region);
    uint16_t* dout = reinterpret_cast<uint16_t*>(region + code_bytes);
    // update and in-lane maxima of |x| of the lane's rows, then the row maxima over the
    // 16 lanes of each row reduced and scattered (each lane ends with one of the 4 rows),
    // so that every step is derived once per 4 lanes and handed back by quad broadcasts
    // dequantize + decay from the codes kept as floats (x = code alpha + beta0), then the
    // update
    uint32_t mxb[MR];
    float sab[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const TabA ta = taw[NG * m + rq];
#pragma unroll
        for (int c = 0; c < 8; ++c) x[m][c] = __builtin_fmaf(ta.k, wv[c], __builtin_fmaf(x[m][c], ta.alpha, ta.beta0));
        float mx = fmaxf(fmaxf(fabsf(x[m][0]), fabsf(x[m][1])), fabsf(x[m][2]));
        mx = fmaxf(fmaxf(mx, fabsf(x[m][3])), fabsf(x[m][4]));
        mx = fmaxf(fmaxf(mx, fabsf(x[m][5])), fabsf(x[m][6]));
        mxb[m] = __float_as_uint(fmaxf(mx, fabsf(x[m][7])));
        if constexpr (OB)
            sab[m] = ((fabsf(x[m][0]) + fabsf(x[m][1])) + (fabsf(x[m][2]) + fabsf(x[m][3]))) +
                     ((fabsf(x[m][4]) + fabsf(x[m][5])) + (fabsf(x[m][6]) + fabsf(x[m][7])));
    }
    float inv[MR];
    float dls[MR];                              // error feedback: the rows' steps
    // error feedback: the residuals of the lane's rows, one row ahead of their rounding
    // (the first requested before the steps are derived, so that its latency overlaps it)
    auto eptr_of = [&](int m) {
        return reinterpret_cast<float4*>(A.side + ((size_t)head * DK + tbw[NG * m + rq].row) * DV + 8 * cg);
    };
    float4 epre[2];
    if constexpr (EF) {
        const float4* ep = eptr_of(0);
        epre[0] = ep[0];
        epre[1] = ep[1];
    }
    {
        // this lane's row: ms = ((cg & 1) << 1) | ((cg >> 1) & 1)
        const int ms = ((cg & 1) << 1) | ((cg >> 1) & 1);
        const TabB tb = tbw[NG * ms + rq];
        const float R = __uint_as_float(rowmax4_scatter(mxb, cg));
        uint32_t dbits = f16_bits_of_product(R, tb.fn);
        if constexpr (OB) {
            // one-bit row: Delta = f16(mean |x|), the row sum by a pairwise sum in the lane
            // and four DPP steps (relative error below 7 float32 roundings)
            const float sa = rowsum4_scatter(sab, cg);
            const uint32_t d1 = f16_bits_of_product(sa, 1.f / float(DV));
            if (tb.bw == 1u) dbits = d1;
        }
        const float dl = f16_bits_to_f32(dbits);
        // reciprocal refined by one Newton step (near correctly rounded)
        float r = __builtin_amdgcn_rcpf(dl);
        r = __builtin_fmaf(__builtin_fmaf(-dl, r, 1.f), r, r);
        const uint32_t ib = __float_as_uint(dl > 0.f ? r : 0.f);
        if (cg < 4) dout[tb.row] = uint16_t(dbits);
        // row m sits in quad lane ((m & 1) << 1) | (m >> 1)
        inv[0] = __uint_as_float(dpp_u32<0x00>(ib));
        inv[1] = __uint_as_float(dpp_u32<0xAA>(ib));
        inv[2] = __uint_as_float(dpp_u32<0x55>(ib));
        inv[3] = __uint_as_float(dpp_u32<0xFF>(ib));
        if constexpr (EF) {
            const uint32_t db = __float_as_uint(dl);
            dls[0] = __uint_as_float(dpp_u32<0x00>(db));
            dls[1] = __uint_as_float(dpp_u32<0xAA>(db));
            dls[2] = __uint_as_float(dpp_u32<0x55>(db));
            dls[3] = __uint_as_float(dpp_u32<0xFF>(db));
        }
    }
    // ... then the rounding and packing, specialised per width
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const TabB* tb = &tbw[NG * m + rq];
        if constexpr (EF) {
            float4* ep = eptr_of(m);
            const float4 e0 = epre[0], e1 = epre[1];
            if (m + 1 < MR) {
                const float4* en = eptr_of(m + 1);
                epre[0] = en[0];
                epre[1] = en[1];
            }
            float e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
            uint32_t y[8];
            const int bw = int(tb->bw);
            ef_round8<OB>(x[m], e, inv[m], dls[m], bw, y);
            ep[0] = make_float4(e[0], e[1], e[2], e[3]);
            ep[1] = make_float4(e[4], e[5], e[6], e[7]);
            store_rows<OB>(gout, boff_of(loc_of(m)), bus[m], bw, y);
        } else {
            uint32_t r16[8];
            if constexpr (SR) sr_draws8(A.seed, uint32_t(head), A.t, int(tb->row), cg, r16);
            pack_rows<OB, SR>(gout, boff_of(loc_of(m)), bus[m], &tb->bw, x[m], inv[m], r16);
        }
    }
}

}  // namespace

namespace {
template <bool EST, bool LAYER, bool OB>
void launch_variant(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.mode == WB_SR)
        hipLaunchKernelGGL((bitalloc_step_kernel<EST, LAYER, OB, WB_SR>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else if (d.mode == WB_EF)
        hipLaunchKernelGGL((bitalloc_step_kernel<EST, LAYER, OB, WB_EF>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
    else
        hipLaunchKernelGGL((bitalloc_step_kernel<EST, LAYER, OB, WB_RTN>), dim3(d.B * d.H), dim3(NT), 0, stream, a);
}
template <bool EST, bool LAYER>
void launch_ob(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.bmin == 1) launch_variant<EST, LAYER, true>(d, a, stream);
    else launch_variant<EST, LAYER, false>(d, a, stream);
}
template <bool EST>
void launch_layer(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (a.layer) launch_ob<EST, true>(d, a, stream);
    else launch_ob<EST, false>(d, a, stream);
}
}  // namespace

bool bitalloc_step_supported(const wb_layout_desc& d) {
    return d.dk == DK && d.dv == DV && (d.mode == WB_RTN || d.mode == WB_SR || d.mode == WB_EF) && d.bmin >= 1 &&
           d.bmax <= 8 && (d.budget == WB_BUDGET_HEAD || d.budget == WB_BUDGET_LAYER);
}

// ---------------------------------------------------------------------------
// Decode write-back step of the per-head allocation unit (HEADALLOC) with round to
// nearest, stochastic rounding or error feedback ([LBRS] "Allocation units"): one width b for the whole head, and a float16 step
// per group of 32 key rows and value column with its own fit index. Four wavefronts per
// head, one per row group: lane (cg, rq) of wavefront g holds rows 32 g + 8 rq .. + 7 and
// columns 8 cg .. 8 cg + 7, so a column's group maximum is the maximum over the lane's 8
// rows and the 4 lanes 16 apart, and every step a lane reads or rounds with belongs to
// its own group. The width is the same for every row of a head, so the body is
// specialised per width and chosen once per workgroup.
namespace {

constexpr int HNW = 4, HNT = 64 * HNW;         // one wavefront per row group
constexpr int HGR = DK / 32;                   // row groups
constexpr int HMR = 8;                         // rows per lane
constexpr int kHaCodeMax = DK * DV;            // code bytes at 8 bits per value

struct HaSmem {
    float4 row[DK];                             // a_i, k_i a_i, q_i a_i, k_i
    float2 g[HGR * DV];                         // stored Delta and -n Delta per (group, column)
    float fn[HGR * DV];                         // f / n per (group, column)
    float ginv[HGR * DV];                       // 1 / new Delta (0 for a zero step)
    float red[2][HNW][DV];                      // u / p partials of the wavefronts
    float w[DV];
    float qk[2];
    alignas(16) uint32_t reg[kHaCodeMax / 4 + 4];   // staged codes (+16 bytes a row's 3-word read may touch)
};

template <int B, int RULE>
__device__ __forceinline__ void headalloc_body(const KArgs& A, HaSmem& sm) {
    constexpr bool SR = RULE == WB_SR, EF = RULE == WB_EF;
    constexpr int n = (1 << (B - 1)) - 1;
    constexpr int NVEC = DK * DV * B / 8 / 16;           // 16-byte vectors of codes in use
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = blockIdx.x;
    const int cg = lane & 15, rq = lane >> 4;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int cap = A.code_cap;
    const uint4* src = reinterpret_cast<const uint4*>(region);

    // Wavefronts 0 and 1 load the per-row inputs and the stored steps and fit bytes and
    // build the tables (at a raised issue priority: the rest of the workgroup waits for
    // them); wavefronts 2 and 3 copy the codes into LDS with global-to-LDS loads, so
    // that neither pair's waits include the other's loads.
    float vj = 0.f, beta = 0.f;
    if (wave < 2) {
        vj = A.v[(size_t)head * DV + tid];
        beta = A.beta[head];
        const size_t rb = (size_t)head * DK + tid;
        const float kr = A.k[rb], qr = A.q[rb];
        const float sr = A.s_per_row ? A.s[rb] : A.s[head];
        uint32_t dbits[4], fbyte[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tid + 2 * 64 * i;
            dbits[i] = reinterpret_cast<const uint16_t*>(region + cap)[t];
            fbyte[i] = region[cap + 2 * HGR * DV + t];
        }
        __builtin_amdgcn_s_setprio(3);
        // per-row constants and q . k
        if (A.est) ema_fold_row(A.est + (size_t)head * est_stride(DK), DK, tid, sr, beta, kr);
        const float a = expf(-sr);
        sm.row[tid] = make_float4(a, kr * a, qr * a, kr);
        float pq = qr * kr;
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0xB1, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x4E, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x141, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x140, 0xF, 0xF, false));
        const float qsum = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 0)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 16))) +
                           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 32)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 48)));
        if (lane == 0) sm.qk[wave] = qsum;
        // stored steps and fit fractions per (group, column): thread owns t = tid + 128 i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tid + 2 * 64 * i;
            const float dold = f16_bits_to_f32(dbits[i]);
            sm.g[t] = make_float2(dold, -float(n) * dold);     // exact: 11 + 7 significant bits
            sm.fn[t] = fn_of(int(fbyte[i] & 15u), B);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        // vectors i0 + lane of the codes, i0 = 64 (wave - 2) + 128 r (a scalar)
        for (int i0 = 64 * (wave - 2); i0 < NVEC; i0 += 128) lds_load16(src + i0 + lane, &sm.reg[4 * i0]);
        lds_loads_wait();
    }
    __syncthreads();

    // ---- dequantize the lane's 8 rows x 8 columns (group `wave`); u, p partials -------
    // x0 = Delta (code - n) is exact; the decay is folded into the row weights of u and
    // p and into the update.
    const int row0 = 32 * wave + HMR * rq;
    float gd[8], gn[8];
    {
        const float4* gp = reinterpret_cast<const float4*>(&sm.g[wave * DV + 8 * cg]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = gp[i];
            gd[2 * i] = v.x;
            gn[2 * i] = v.y;
            gd[2 * i + 1] = v.z;
            gn[2 * i + 1] = v.w;
        }
    }
    float x[HMR][8], up[8], pp[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        up[c] = 0.f;
        pp[c] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < HMR; ++m) {
        const int boff = (row0 + m) * (DV / 8) * B + cg * B;
        float code[8];
        unpack8<B>(load_raw(sm.reg, boff), boff, code);
        const float4 tr = sm.row[row0 + m];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            x[m][c] = __builtin_fmaf(code[c], gd[c], gn[c]);
            up[c] = __builtin_fmaf(tr.y, x[m][c], up[c]);
            pp[c] = __builtin_fmaf(tr.z, x[m][c], pp[c]);
        }
    }
    // the four row blocks of the wavefront summed by lane swaps (as in the per-row
    // kernel): lane (cg, rq) then holds quantity rq / 2 of columns 8 cg + 4 (rq % 2) + 0..3
    {
        float t[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(up[c]), __float_as_uint(pp[c]), false,
                                                            false);
            t[c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        float s4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t[c]), __float_as_uint(t[c + 4]), false,
                                                            false);
            s4[c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        *reinterpret_cast<float4*>(&sm.red[rq >> 1][wave][8 * cg + 4 * (rq & 1)]) =
            make_float4(s4[0], s4[1], s4[2], s4[3]);
    }
    __syncthreads();

    // ---- w = beta (v - u) (threads 0..127); p summed by threads 128..255 for o --------
    const int jq = tid >> 7, j = tid & (DV - 1);
    float pj = 0.f;
    {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < HNW; ++g) acc += sm.red[jq][g][j];
        if (jq == 0) sm.w[j] = beta * (vj - acc);
        else pj = acc;
    }
    __syncthreads();
    if (jq == 1) A.o[(size_t)head * DV + j] = __builtin_fmaf(sm.qk[0] + sm.qk[1], sm.w[j], pj);

    // ---- update and group maxima ---------------------------------------------------------
    float wv[8], mx[8];
    {
        const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[8 * cg]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[8 * cg + 4]);
        wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
        wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) mx[c] = 0.f;
#pragma unroll
    for (int m = 0; m < HMR; ++m) {
        const float4 tr = sm.row[row0 + m];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            x[m][c] = __builtin_fmaf(tr.x, x[m][c], tr.w * wv[c]);
            mx[c] = fmaxf(mx[c], fabsf(x[m][c]));
        }
    }
    // over the group's other rows: the lanes 16 and 32 apart
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx[c]), __float_as_uint(mx[c]), false, false);
        const float v = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        mx[c] = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
    // new steps: lane (cg, rq) derives columns 8 cg + 2 rq and 8 cg + 2 rq + 1
    {
        float R0 = mx[0], R1 = mx[1];
        if (rq == 1) { R0 = mx[2]; R1 = mx[3]; }
        if (rq == 2) { R0 = mx[4]; R1 = mx[5]; }
        if (rq == 3) { R0 = mx[6]; R1 = mx[7]; }
        uint16_t* dnew = reinterpret_cast<uint16_t*>(region + cap);     // straight to HBM
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int t = wave * DV + 8 * cg + 2 * rq + e;
            const uint32_t dbits = f16_bits_of_product(e ? R1 : R0, sm.fn[t]);
            const float dl = f16_bits_to_f32(dbits);
            float r = __builtin_amdgcn_rcpf(dl);
            r = __builtin_fmaf(__builtin_fmaf(-dl, r, 1.f), r, r);
            sm.ginv[t] = dl > 0.f ? r : 0.f;
            // error feedback: the new step itself, in the slot of the stored one (read
            // only by the unpack, before the partial-sum barrier)
            if constexpr (EF) sm.g[t].x = dl;
            dnew[t] = uint16_t(dbits);
        }
    }
    __syncthreads();

    // ---- round on each column's grid and pack; each lane stores its codes in HBM --------
    uint32_t* gout = reinterpret_cast<uint32_t*>(region);
    float gi[8];
    {
        const float4 i0 = *reinterpret_cast<const float4*>(&sm.ginv[wave * DV + 8 * cg]);
        const float4 i1 = *reinterpret_cast<const float4*>(&sm.ginv[wave * DV + 8 * cg + 4]);
        gi[0] = i0.x; gi[1] = i0.y; gi[2] = i0.z; gi[3] = i0.w;
        gi[4] = i1.x; gi[5] = i1.y; gi[6] = i1.z; gi[7] = i1.w;
    }
    float gdl[8];
    if constexpr (EF) {
#pragma unroll
        for (int c = 0; c < 8; ++c) gdl[c] = sm.g[wave * DV + 8 * cg + c].x;
    }
#pragma unroll
    for (int m = 0; m < HMR; ++m) {
        const int boff = (row0 + m) * (DV / 8) * B + cg * B;
        if constexpr (EF) {
            // error feedback: y + e to the nearest level of the column's grid, the residual
            // y + e - level Delta clipped to one step (a zero step: level 0, residual 0)
            float4* ep = reinterpret_cast<float4*>(A.side + ((size_t)head * DK + row0 + m) * DV + 8 * cg);
            const float4 e0 = ep[0], e1 = ep[1];
            float e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
            uint32_t y[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float t = x[m][c] + e[c];
                const float yf = __builtin_amdgcn_fmed3f(__builtin_fmaf(t, gi[c], kMagic), kMagic - float(n),
                                                         kMagic + float(n));
                y[c] = __float_as_uint(yf);
                e[c] = fminf(fmaxf(t - (yf - kMagic) * gdl[c], -gdl[c]), gdl[c]);
            }
            ep[0] = make_float4(e[0], e[1], e[2], e[3]);
            ep[1] = make_float4(e[4], e[5], e[6], e[7]);
            store8<B>(gout, boff, y);
        } else if constexpr (SR) {
            // stochastic rounding with the element's Philox draws (row, column group)
            uint32_t r16[8], y[8];
            sr_draws8(A.seed, uint32_t(head), A.t, row0 + m, cg, r16);
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] = sr_field<B>(x[m][c], gi[c], gi[c] * -65536.f, r16[c]);
            store8<B, true>(gout, boff, y);
        } else {
            pack8<B>(gout, boff, x[m], InvCol{gi});
        }
    }
    // (the fit bytes and the width byte are unchanged)
}

template <int RULE>
__global__ void __launch_bounds__(HNT) headalloc_step_kernel(const KArgs A) {
    __shared__ HaSmem sm;
    const uint8_t* region = A.state + (size_t)blockIdx.x * A.region_stride;
    // the head's width byte follows the steps and fit indices; kept inside [2, b_max]
    int b = int(region[A.code_cap + 3 * HGR * DV]) + 1;
    b = __builtin_amdgcn_readfirstlane(min(max(b, 2), A.code_cap / (DK * DV / 8)));
    switch (b) {
        case 2: headalloc_body<2, RULE>(A, sm); break;
        case 3: headalloc_body<3, RULE>(A, sm); break;
        case 4: headalloc_body<4, RULE>(A, sm); break;
        case 5: headalloc_body<5, RULE>(A, sm); break;
        case 6: headalloc_body<6, RULE>(A, sm); break;
        case 7: headalloc_body<7, RULE>(A, sm); break;
        default: headalloc_body<8, RULE>(A, sm); break;
    }
}

}  // namespace

bool headalloc_step_supported(const wb_layout_desc& d) {
    return d.kind == WB_HEADALLOC && d.dk == DK && d.dv == DV &&
           (d.mode == WB_RTN || d.mode == WB_SR || d.mode == WB_EF) && d.bmax <= 8;
}

hipError_t launch_headalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.mode == WB_SR) hipLaunchKernelGGL(headalloc_step_kernel<WB_SR>, dim3(d.B * d.H), dim3(HNT), 0, stream, a);
    else if (d.mode == WB_EF) {
        if (a.side == nullptr) return hipErrorInvalidValue;
        hipLaunchKernelGGL(headalloc_step_kernel<WB_EF>, dim3(d.B * d.H), dim3(HNT), 0, stream, a);
    } else hipLaunchKernelGGL(headalloc_step_kernel<WB_RTN>, dim3(d.B * d.H), dim3(HNT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bitalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    // the staged region: the code area (per head: b-bar bits per element; layer budget:
    // b_max), Delta and the width / fit bytes
    const size_t code_area = size_t(a.layer ? a.code_cap : DK * DV * d.bbar / 8);
    if (code_area > size_t(kCodeAreaMax)) return hipErrorInvalidValue;
    if (d.mode == WB_EF && a.side == nullptr) return hipErrorInvalidValue;
    if (a.est) launch_layer<true>(d, a, stream);
    else launch_layer<false>(d, a, stream);
    return hipGetLastError();
}

}  // namespace wb
