// Decode write-back step for the decay-aware per-row-width layout (BITALLOC), tuned for
// the VALU budget of gfx950.
//
// Same computation as the generic decode kernel (dequantize -> decay -> u = k^T D S ->
// w = beta (v - u) -> S' = D S + k w^T -> o -> Delta_i = f16(f_i R_i / n_i) -> nearest
// level -> pack), organised so that each stored element costs few vector instructions:
//   * rows are visited in order of increasing width, so the 4 rows a wavefront handles
//     per step nearly always share one width; that width is read into a scalar register
//     and the unpack / pack code is chosen by a scalar branch and specialised per width
//     (static bit positions); a group of mixed widths is walked one width at a time;
//   * eight wavefronts per head; a lane holds 4 rows x 8 columns of the state (32
//     values, which keeps the register count low enough for 6 wavefronts per SIMD), and
//     the u / p partial sums of a wavefront are combined in registers by lane swaps
//     before one LDS store;
//   * the sort, the byte offsets of the rows and their ranks come from wavefront ballots
//     (each of the two wavefronts that build the tables reads the widths of all 128
//     rows, so no cross-wave scan is needed);
//   * per-row constants (decayed step, offset term, k_i, q_i, f_i / n_i, rounding
//     constants, byte offset, width) sit in LDS tables indexed by sorted position;
//   * dequantize + decay is one FMA: a_i Delta_i (code - n_i) = code * (a_i Delta_i) +
//     (-n_i a_i Delta_i);
//   * rounding to the nearest level adds 1.5 * 2^23 + n_i in the same FMA as the scaling
//     (x * (1/Delta) + magic rounds the exact product once, ties to even), clamps with
//     one med3, and packs with shift-adds whose constant high bits are removed once per
//     32-bit word;
//   * row maxima use DPP integer max on the bits of |x| (ordered like the values);
//   * the packed codes of a lane (8 elements = b bytes) go to a staging copy of the
//     region in LDS at their final byte offset, then the region is written to HBM with
//     16-byte stores.
// Two more instantiations widen it: the layer-wise budget (the code area holds every
// row at b_max; the widths are read first and only the codes in use are staged and
// written back, so the zero tail is never touched) and one-bit rows (the two levels
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
    float fn;                                   // f / n
    uint32_t loc;                               // byte offset | width << 16 | row << 24
};

struct BaFixed {
    TabA ta[DK];
    TabB tb[DK];
    float red[2][NW][DV];                      // u / p partials of the wavefronts
    float w[DV];
    float qk[4];
};
// the staged region follows BaFixed in dynamic LDS
constexpr int kRegOffset = (int(sizeof(BaFixed)) + 15) / 16 * 16;

// f_k / n_b for fit index k (f_k = 1/4 + k/20) and width b (n_b = 2^(b-1) - 1)
struct FnTable {
    float v[16][9];
    constexpr FnTable() : v() {
        for (int k = 0; k < 16; ++k)
            for (int b = 2; b <= 8; ++b) v[k][b] = (0.25f + 0.05f * float(k)) / float((1 << (b - 1)) - 1);
    }
};
__constant__ FnTable kFn = FnTable();

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

// Write 8 codes of `B` bits, given in magic-number form (the bits of 1.5 * 2^23 + code),
// packed at byte `boff` of the staging copy (B bytes).
template <int B>
__device__ __forceinline__ void store8(uint32_t* reg, int boff, const uint32_t y[8]) {
    if constexpr (B == 1) {
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) w |= (y[c] - kMagicBits) << c;
        reinterpret_cast<uint8_t*>(reg)[boff] = uint8_t(w);
        return;
    }
    // the constant high bits of every shifted y are removed once per word
    uint32_t g0 = 0, g1 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int p = c * B;
        if (p + B <= 32) g0 += kMagicBits << p;
        else if (p >= 32) g1 += kMagicBits << (p - 32);
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
            const uint32_t code = y[c] - kMagicBits;
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
        for (int i = 0; i < B; ++i) bytes[boff + i] = uint8_t(i < 4 ? (w0 >> (8 * i)) : (w1 >> (8 * (i - 4))));
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
        constexpr float n = float((1 << (B - 1)) - 1);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            y[c] = __float_as_uint(
                __builtin_amdgcn_fmed3f(__builtin_fmaf(x[c], inv[c], kMagic + n), kMagic, kMagic + 2.f * n));
    }
    store8<B>(reg, boff, y);
}

// Stochastic rounding of one value on the grid of the row (level index in [0, 2n], or
// [0, 1] for a one-bit row on -Delta + k 2 Delta): floor(tau) + [u < frac(tau)] with u the
// 16-bit draw over 2^16, clamped at the rails; a zero step stores level 0 (offset n).
__device__ __forceinline__ uint32_t sr_level(float x, float inv, int bw, uint32_t r16) {
    const bool one = bw == 1;
    const float n = one ? 0.f : float((1 << (bw - 1)) - 1);
    const float tau = one ? (inv > 0.f ? __builtin_fmaf(x, 0.5f * inv, 0.5f) : 0.f) : x * inv;
    const float fl = floorf(tau);
    float k = fl + ((float(r16) < (tau - fl) * 65536.f) ? 1.f : 0.f);
    k = one ? __builtin_amdgcn_fmed3f(k, 0.f, 1.f) : __builtin_amdgcn_fmed3f(k, -n, n);
    return __float_as_uint(kMagic + (k + n));
}

template <int B>
__device__ __forceinline__ void pack8_sr(uint32_t* reg, int boff, const float x[8], float inv, const uint32_t r16[8]) {
    uint32_t y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = sr_level(x[c], inv, B, r16[c]);
    store8<B>(reg, boff, y);
}

// Generic unpack / pack for a per-lane width (a group of rows of mixed widths).
__device__ __forceinline__ void unpack8_any(const Raw& raw, int boff, int bw, float code[8]) {
    const int sh = (boff & 3) * 8;
    const uint32_t lo = __builtin_amdgcn_alignbit(raw.w1, raw.w0, sh);
    const uint32_t hi = __builtin_amdgcn_alignbit(raw.w2, raw.w1, sh);
    const uint64_t fld = uint64_t(lo) | (uint64_t(hi) << 32);
    const uint32_t mask = (1u << bw) - 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) code[c] = float(uint32_t(fld >> (c * bw)) & mask);
}

template <bool OB, bool SR>
__device__ __forceinline__ void pack8_any(uint32_t* reg, int boff, int bw, const float x[8], float inv,
                                          const uint32_t r16[8]) {
    const float n = float((1 << (bw - 1)) - 1);
    uint64_t fld = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t code;
        if constexpr (SR) {
            code = sr_level(x[c], inv, bw, r16[c]) - kMagicBits;
        } else {
            const uint32_t y = __float_as_uint(
                __builtin_amdgcn_fmed3f(__builtin_fmaf(x[c], inv, kMagic + n), kMagic, kMagic + 2.f * n));
            code = y - kMagicBits;
            if (OB && bw == 1) code = x[c] * inv > 0.f;
        }
        fld |= uint64_t(code) << (c * bw);
    }
    uint8_t* bytes = reinterpret_cast<uint8_t*>(reg);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < bw) bytes[boff + i] = uint8_t(fld >> (8 * i));
}

// Unpack / pack with the width held per lane. When the lanes share one width (rows
// handled together are adjacent in the width order, so this is the common case), the
// width is a scalar and the specialised code is chosen by a scalar branch; otherwise
// the generic per-lane code runs.
template <bool OB>
__device__ __forceinline__ void unpack_rows(const Raw& raw, int boff, int bw, float code[8]) {
    const int bu = __builtin_amdgcn_readfirstlane(bw);
    if (__ballot(bw != bu) == 0ull) {
        if (OB && bu == 1) {
            unpack8<1>(raw, boff, code);
            return;
        }
        switch (bu) {
            case 2: unpack8<2>(raw, boff, code); break;
            case 3: unpack8<3>(raw, boff, code); break;
            case 4: unpack8<4>(raw, boff, code); break;
            case 5: unpack8<5>(raw, boff, code); break;
            case 6: unpack8<6>(raw, boff, code); break;
            case 7: unpack8<7>(raw, boff, code); break;
            default: unpack8<8>(raw, boff, code); break;
        }
    } else {
        unpack8_any(raw, boff, bw, code);
    }
}

template <int B, bool SR>
__device__ __forceinline__ void pack8_rule(uint32_t* reg, int boff, const float x[8], float inv, const uint32_t r16[8]) {
    if constexpr (SR) pack8_sr<B>(reg, boff, x, inv, r16);
    else pack8<B>(reg, boff, x, InvOne{inv});
}

template <bool OB, bool SR>
__device__ __forceinline__ void pack_rows(uint32_t* reg, int boff, int bw, const float x[8], float inv,
                                          const uint32_t r16[8]) {
    const int bu = __builtin_amdgcn_readfirstlane(bw);
    if (__ballot(bw != bu) == 0ull) {
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
        pack8_any<OB, SR>(reg, boff, bw, x, inv, r16);
    }
}

// max over the 16 lanes of a DPP row, of non-negative floats given as bit patterns
__device__ __forceinline__ uint32_t rowmax16_bits(uint32_t v) {
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));   // xor 1
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));   // xor 2
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));  // half mirror
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));  // mirror
    return v;
}

// sum over the 16 lanes of a DPP row (the same butterfly as the maximum)
__device__ __forceinline__ float rowsum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
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

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// EST: fold the token into the attached online estimators; LAYER: the layer-wise budget
// layout (code area of b_max bits per element, codes in use first, then a zero tail);
// OB: one-bit rows may occur; SR: stochastic rounding with the Philox draws of the
// element (row, 8 columns) instead of round to nearest. Each is its own instantiation, so that the plain step
// carries no trace of the others.
template <bool EST, bool LAYER, bool OB, bool SR>
__global__ void __launch_bounds__(NT) bitalloc_step_kernel(const KArgs A) {
    extern __shared__ __align__(16) uint8_t smraw[];
    BaFixed& sm = *reinterpret_cast<BaFixed*>(smraw);
    uint32_t* reg = reinterpret_cast<uint32_t*>(smraw + kRegOffset);
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

    // ---- loads: the region (staged through registers), metadata, per-row inputs ------
    // Per-head budget: the region in one piece. Layer budget: the codes every head holds
    // (b_min bits per element) and the metadata, then, once the widths are summed, the
    // rest of the codes in use.
    uint4 pf0 = make_uint4(0, 0, 0, 0), pf1 = pf0, pf2 = pf0, pfm = pf0;
    const uint4* src = reinterpret_cast<const uint4*>(region);
    int nvec = 0, nmin = 0, ncode = 0;
    int meta0 = 0, meta1 = 0;
    if constexpr (!LAYER) {
        nvec = (code_bytes + 3 * DK) / 16;
        if (tid < nvec) pf0 = src[tid];
        if (tid + NT < nvec) pf1 = src[tid + NT];
        if (tid + 2 * NT < nvec) pf2 = src[tid + 2 * NT];
    } else {
        nmin = min(A.bmin * (DK * DV / 8 / 16), NT);
        if (tid < nmin) pf0 = src[tid];
        if (tid < kMetaVec) pfm = src[code_bytes / 16 + tid];
        meta0 = meta[lane];
        meta1 = meta[lane + 64];
        // 16-byte vectors of codes in use: sum of the widths times DV / 128 (at most the
        // code area)
        ncode = min(wave_sum_i32((meta0 & 7) + (meta1 & 7) + 2) * (DV / 128), code_bytes / 16);
        if (nmin + tid < ncode) pf1 = src[nmin + tid];
        if (nmin + tid + NT < ncode) pf2 = src[nmin + tid + NT];
    }
    const float vj = A.v[(size_t)head * DV + (tid & (DV - 1))];
    const float beta = A.beta[head];

    // ---- per-row tables: wavefronts 0 and 1 own rows lane and lane + 64 ---------------
    // The width order, the byte offsets and the ranks come from ballots over the width
    // bytes of all 128 rows, which both wavefronts read.
    if (wave < 2) {
        if constexpr (!LAYER) {
            meta0 = meta[lane];
            meta1 = meta[lane + 64];
        }
        const int trow = lane + 64 * wave;
        const size_t rb = (size_t)head * DK + trow;
        const float kr = A.k[rb], qr = A.q[rb];
        const float sr = A.s_per_row ? A.s[rb] : A.s[head];
        if constexpr (EST) ema_fold_row(A.est + (size_t)head * est_stride(DK), DK, trow, sr, beta, kr);
        const uint32_t dold = reinterpret_cast<const uint16_t*>(region + code_bytes)[trow];
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
        // a one-bit row's levels are -Delta, +Delta: code * 2 a Delta - a Delta
        if (OB && bwt == 1) sm.ta[pos] = TabA{2.f * ad, -ad, kr, qr};
        else sm.ta[pos] = TabA{ad, -n * ad, kr, qr};
        sm.tb[pos] = TabB{kFn.v[fit][bwt], uint32_t(off * (DV / 8)) | (uint32_t(bwt) << 16) | (uint32_t(trow) << 24)};
        // q . k over the wavefront's 64 rows: DPP sums inside each row of 16 lanes, then
        // the four row sums
        float pq = qr * kr;
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0xB1, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x4E, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x141, 0xF, 0xF, false));
        pq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pq), 0x140, 0xF, 0xF, false));
        // (read the row sums with every lane active; only the store is predicated)
        const float qsum = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 0)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 16))) +
                           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 32)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 48)));
        if (lane == 0) sm.qk[wave] = qsum;
    }
    {
        uint4* dst = reinterpret_cast<uint4*>(reg);
        if constexpr (!LAYER) {
            if (tid < nvec) dst[tid] = pf0;
            if (tid + NT < nvec) dst[tid + NT] = pf1;
            if (tid + 2 * NT < nvec) dst[tid + 2 * NT] = pf2;
        } else {
            if (tid < nmin) dst[tid] = pf0;
            if (tid < kMetaVec) dst[code_bytes / 16 + tid] = pfm;
            if (nmin + tid < ncode) dst[nmin + tid] = pf1;
            if (nmin + tid + NT < ncode) dst[nmin + tid + NT] = pf2;
        }
    }
    __syncthreads();

    // ---- dequantize the lane's 4 rows x 8 columns; u, p partial sums ------------------
    // The code words of row m + 1 are requested (and the location of row m + 2 read)
    // before row m is unpacked, so their LDS latency overlaps the arithmetic.
    auto boff_of = [&](uint32_t l) { return int(l & 0xFFFFu) + cg * int((l >> 16) & 15u); };
    float x[MR][8];
    float up[8], pp[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        up[c] = 0.f;
        pp[c] = 0.f;
    }
    uint32_t loc_cur = sm.tb[4 * wave + rq].loc;
    uint32_t loc_next = sm.tb[NG + 4 * wave + rq].loc;
    Raw raw_next = load_raw(reg, boff_of(loc_cur));
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const Raw raw = raw_next;
        const uint32_t loc = loc_cur;
        if (m + 1 < MR) {
            raw_next = load_raw(reg, boff_of(loc_next));
            loc_cur = loc_next;
        }
        if (m + 2 < MR) loc_next = sm.tb[NG * (m + 2) + 4 * wave + rq].loc;
        const TabA ta = sm.ta[NG * m + 4 * wave + rq];
        float code[8];
        unpack_rows<OB>(raw, boff_of(loc), int((loc >> 16) & 15u), code);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            x[m][c] = __builtin_fmaf(code[c], ta.alpha, ta.beta0);
            up[c] = __builtin_fmaf(ta.k, x[m][c], up[c]);
            pp[c] = __builtin_fmaf(ta.q, x[m][c], pp[c]);
        }
        // finish this row here (keeps the codes of one row live at a time)
        asm volatile("" ::"v"(x[m][0]), "v"(x[m][1]), "v"(x[m][2]), "v"(x[m][3]), "v"(x[m][4]), "v"(x[m][5]),
                     "v"(x[m][6]), "v"(x[m][7]));
        asm volatile("" ::"v"(up[0]), "v"(up[1]), "v"(up[2]), "v"(up[3]), "v"(up[4]), "v"(up[5]), "v"(up[6]),
                     "v"(up[7]), "v"(pp[0]), "v"(pp[1]), "v"(pp[2]), "v"(pp[3]), "v"(pp[4]), "v"(pp[5]), "v"(pp[6]),
                     "v"(pp[7]));
    }
    // Sum the four row groups of the wavefront in registers (a reduce-scatter by lane
    // swaps): exchanging lanes 32..63 of u with lanes 0..31 of p and adding leaves the
    // u sums over row groups (0, 2) and (1, 3) in the low half and the p sums in the
    // high half; exchanging odd 16-lane rows of columns c with even rows of columns
    // c + 4 and adding completes the sums. Lane (cg, rq) then holds quantity rq / 2 of
    // columns 8 cg + 4 (rq % 2) + 0..3.
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
    if (jq < 2) {
        float acc = 0.f;
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

    // ---- update and requantize into the staging copy -----------------------------------
    float wv[8];
    {
        const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[8 * cg]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[8 * cg + 4]);
        wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
        wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
    }
    uint16_t* dout = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(reg) + code_bytes);
    // row maxima and steps first (no branches, so the lane's rows interleave) ...
    float inv[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int pos = NG * m + 4 * wave + rq;
        const float kk = sm.ta[pos].k;
        const TabB tb = sm.tb[pos];
#pragma unroll
        for (int c = 0; c < 8; ++c) x[m][c] = __builtin_fmaf(kk, wv[c], x[m][c]);
        float mx = fmaxf(fmaxf(fabsf(x[m][0]), fabsf(x[m][1])), fabsf(x[m][2]));
        mx = fmaxf(fmaxf(mx, fabsf(x[m][3])), fabsf(x[m][4]));
        mx = fmaxf(fmaxf(mx, fabsf(x[m][5])), fabsf(x[m][6]));
        mx = fmaxf(mx, fabsf(x[m][7]));
        const float R = __uint_as_float(rowmax16_bits(__float_as_uint(mx)));
        uint32_t dbits = f16_bits_of_product(R, tb.fn);
        if constexpr (OB) {
            // one-bit row: Delta = f16(mean |x|), the row sum by a pairwise sum in the lane
            // and a DPP butterfly (relative error below 7 float32 roundings)
            const bool one = ((tb.loc >> 16) & 15u) == 1u;
            if (__ballot(one) != 0ull) {
                float sa = ((fabsf(x[m][0]) + fabsf(x[m][1])) + (fabsf(x[m][2]) + fabsf(x[m][3]))) +
                           ((fabsf(x[m][4]) + fabsf(x[m][5])) + (fabsf(x[m][6]) + fabsf(x[m][7])));
                sa = rowsum16(sa);
                const uint32_t d1 = f16_bits_of_product(sa, 1.f / float(DV));
                if (one) dbits = d1;
            }
        }
        const float dl = f16_bits_to_f32(dbits);
        // reciprocal refined by one Newton step (near correctly rounded)
        float r = __builtin_amdgcn_rcpf(dl);
        r = __builtin_fmaf(__builtin_fmaf(-dl, r, 1.f), r, r);
        inv[m] = dl > 0.f ? r : 0.f;
        if (cg == 0) dout[tb.loc >> 24] = uint16_t(dbits);
    }
    // ... then the rounding and packing, specialised per width
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint32_t l = sm.tb[NG * m + 4 * wave + rq].loc;
        uint32_t r16[8];
        if constexpr (SR) sr_draws8(A.seed, uint32_t(head), A.t, int(l >> 24), cg, r16);
        pack_rows<OB, SR>(reg, boff_of(l), int((l >> 16) & 15u), x[m], inv[m], r16);
    }
    __syncthreads();
    {
        uint4* dst = reinterpret_cast<uint4*>(region);
        const uint4* lsrc = reinterpret_cast<const uint4*>(reg);
        if constexpr (!LAYER) {
            const int out_vec = (code_bytes + 2 * DK) / 16;
            for (int i = tid; i < out_vec; i += NT) dst[i] = lsrc[i];
        } else {
            // the codes in use, then Delta (the tail and the width / fit bytes are unchanged)
            for (int i = tid; i < ncode + 2 * DK / 16; i += NT) {
                const int vi = i < ncode ? i : code_bytes / 16 + (i - ncode);
                dst[vi] = lsrc[vi];
            }
        }
    }
}

}  // namespace

namespace {
template <bool EST, bool LAYER, bool OB>
void launch_variant(const wb_layout_desc& d, const KArgs& a, size_t smem, hipStream_t stream) {
    if (d.mode == WB_SR)
        hipLaunchKernelGGL((bitalloc_step_kernel<EST, LAYER, OB, true>), dim3(d.B * d.H), dim3(NT), smem, stream, a);
    else
        hipLaunchKernelGGL((bitalloc_step_kernel<EST, LAYER, OB, false>), dim3(d.B * d.H), dim3(NT), smem, stream, a);
}
template <bool EST, bool LAYER>
void launch_ob(const wb_layout_desc& d, const KArgs& a, size_t smem, hipStream_t stream) {
    if (d.bmin == 1) launch_variant<EST, LAYER, true>(d, a, smem, stream);
    else launch_variant<EST, LAYER, false>(d, a, smem, stream);
}
template <bool EST>
void launch_layer(const wb_layout_desc& d, const KArgs& a, size_t smem, hipStream_t stream) {
    if (a.layer) launch_ob<EST, true>(d, a, smem, stream);
    else launch_ob<EST, false>(d, a, smem, stream);
}
}  // namespace

bool bitalloc_step_supported(const wb_layout_desc& d) {
    return d.dk == DK && d.dv == DV && (d.mode == WB_RTN || d.mode == WB_SR) && d.bmin >= 1 && d.bmax <= 8 &&
           (d.budget == WB_BUDGET_HEAD || d.budget == WB_BUDGET_LAYER);
}

// ---------------------------------------------------------------------------
// Decode write-back step of the per-head allocation unit (HEADALLOC) with round to
// nearest or stochastic rounding ([LBRS] "Allocation units"): one width b for the whole head, and a float16 step
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
    uint32_t reg[(kHaCodeMax + 2 * HGR * DV) / 4 + 4];   // staged codes, then the new Delta bits
};

template <int B, bool SR>
__device__ __forceinline__ void headalloc_body(const KArgs& A, HaSmem& sm) {
    constexpr int n = (1 << (B - 1)) - 1;
    constexpr int NVEC = DK * DV * B / 8 / 16;           // 16-byte vectors of codes in use
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = blockIdx.x;
    const int cg = lane & 15, rq = lane >> 4;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int cap = A.code_cap;
    const uint4* src = reinterpret_cast<const uint4*>(region);

    uint4 pf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = (tid + HNT * i < NVEC) ? src[tid + HNT * i] : make_uint4(0, 0, 0, 0);
    const float vj = A.v[(size_t)head * DV + (tid & (DV - 1))];
    const float beta = A.beta[head];

    // per-row constants (wavefronts 0 and 1) and q . k
    if (tid < DK) {
        const size_t rb = (size_t)head * DK + tid;
        const float kr = A.k[rb], qr = A.q[rb];
        const float sr = A.s_per_row ? A.s[rb] : A.s[head];
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
    }
    // stored steps and fit fractions per (group, column): thread owns t and t + 256
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = tid + HNT * i;
        const float dold = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(region + cap)[t]);
        const int fit = region[cap + 2 * HGR * DV + t] & 15;
        sm.g[t] = make_float2(dold, -float(n) * dold);     // exact: 11 + 7 significant bits
        sm.fn[t] = kFn.v[fit][B];
    }
    {
        uint4* dst = reinterpret_cast<uint4*>(sm.reg);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tid + HNT * i < NVEC) dst[tid + HNT * i] = pf[i];
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
        uint16_t* dnew = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(sm.reg) + kHaCodeMax);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int t = wave * DV + 8 * cg + 2 * rq + e;
            const uint32_t dbits = f16_bits_of_product(e ? R1 : R0, sm.fn[t]);
            const float dl = f16_bits_to_f32(dbits);
            float r = __builtin_amdgcn_rcpf(dl);
            r = __builtin_fmaf(__builtin_fmaf(-dl, r, 1.f), r, r);
            sm.ginv[t] = dl > 0.f ? r : 0.f;
            dnew[t] = uint16_t(dbits);
        }
    }
    __syncthreads();

    // ---- round to nearest on each column's grid and pack into the staging copy ---------
    float gi[8];
    {
        const float4 i0 = *reinterpret_cast<const float4*>(&sm.ginv[wave * DV + 8 * cg]);
        const float4 i1 = *reinterpret_cast<const float4*>(&sm.ginv[wave * DV + 8 * cg + 4]);
        gi[0] = i0.x; gi[1] = i0.y; gi[2] = i0.z; gi[3] = i0.w;
        gi[4] = i1.x; gi[5] = i1.y; gi[6] = i1.z; gi[7] = i1.w;
    }
#pragma unroll
    for (int m = 0; m < HMR; ++m) {
        const int boff = (row0 + m) * (DV / 8) * B + cg * B;
        if constexpr (SR) {
            // stochastic rounding with the element's Philox draws (row, column group)
            uint32_t r16[8], y[8];
            sr_draws8(A.seed, uint32_t(head), A.t, row0 + m, cg, r16);
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] = sr_level(x[m][c], gi[c], B, r16[c]);
            store8<B>(sm.reg, boff, y);
        } else {
            pack8<B>(sm.reg, boff, x[m], InvCol{gi});
        }
    }
    __syncthreads();

    // ---- the codes, then the new steps (the fit bytes and the width byte are unchanged)
    {
        uint4* dst = reinterpret_cast<uint4*>(region);
        const uint4* ls = reinterpret_cast<const uint4*>(sm.reg);
        constexpr int NOUT = NVEC + 2 * HGR * DV / 16;
        for (int i = tid; i < NOUT; i += HNT) {
            if (i < NVEC) dst[i] = ls[i];
            else dst[cap / 16 + (i - NVEC)] = ls[kHaCodeMax / 16 + (i - NVEC)];
        }
    }
}

template <bool SR>
__global__ void __launch_bounds__(HNT) headalloc_step_kernel(const KArgs A) {
    __shared__ HaSmem sm;
    const uint8_t* region = A.state + (size_t)blockIdx.x * A.region_stride;
    // the head's width byte follows the steps and fit indices; kept inside [2, b_max]
    int b = int(region[A.code_cap + 3 * HGR * DV]) + 1;
    b = __builtin_amdgcn_readfirstlane(min(max(b, 2), A.code_cap / (DK * DV / 8)));
    switch (b) {
        case 2: headalloc_body<2, SR>(A, sm); break;
        case 3: headalloc_body<3, SR>(A, sm); break;
        case 4: headalloc_body<4, SR>(A, sm); break;
        case 5: headalloc_body<5, SR>(A, sm); break;
        case 6: headalloc_body<6, SR>(A, sm); break;
        case 7: headalloc_body<7, SR>(A, sm); break;
        default: headalloc_body<8, SR>(A, sm); break;
    }
}

}  // namespace

bool headalloc_step_supported(const wb_layout_desc& d) {
    return d.kind == WB_HEADALLOC && d.dk == DK && d.dv == DV && (d.mode == WB_RTN || d.mode == WB_SR) &&
           d.bmax <= 8;
}

hipError_t launch_headalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    if (d.mode == WB_SR) hipLaunchKernelGGL(headalloc_step_kernel<true>, dim3(d.B * d.H), dim3(HNT), 0, stream, a);
    else hipLaunchKernelGGL(headalloc_step_kernel<false>, dim3(d.B * d.H), dim3(HNT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bitalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    // the staged region: the code area (per head: b-bar bits per element; layer budget:
    // b_max), Delta and the width / fit bytes
    const size_t code_area = size_t(a.layer ? a.code_cap : DK * DV * d.bbar / 8);
    const size_t smem = kRegOffset + (code_area + 3 * DK + 15) / 16 * 16 + 16;
    if (a.est) launch_layer<true>(d, a, smem, stream);
    else launch_layer<false>(d, a, smem, stream);
    return hipGetLastError();
}

}  // namespace wb
