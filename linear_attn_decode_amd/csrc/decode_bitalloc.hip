// Decode write-back step for the decay-aware per-row-width layout (BITALLOC), tuned for
// the VALU budget of gfx950.
//
// Same computation as the generic decode kernel (dequantize -> decay -> u = k^T D S ->
// w = beta (v - u) -> S' = D S + k w^T -> o -> Delta_i = f16(f_i R_i / n_i) -> nearest
// level -> pack), organised so that each stored element costs few vector instructions:
//   * rows are visited in order of increasing width (a counting sort in the prologue),
//     so the 4 rows a wavefront handles per step nearly always share one width: the
//     unpack and pack code is specialised per width (static bit positions, aligned LDS
//     accesses for 2/4/8-bit rows) and branches are wavefront-uniform;
//   * per-row constants (byte offset, decayed step, offset term, k_i, q_i, f_i / n_i)
//     are computed once per row, not once per lane;
//   * dequantize + decay is one FMA: a_i Delta_i (code - n_i) = code * (a_i Delta_i) +
//     (-n_i a_i Delta_i);
//   * rounding to the nearest level adds 1.5 * 2^23 + n_i in the same FMA as the scaling
//     (x * (1/Delta) + magic rounds the exact product once, ties to even), clamps with
//     one integer med3 on the bit pattern, and packs with shift-adds whose constant
//     high bits are removed once per 32-bit word;
//   * the packed codes of a lane (8 elements = b bytes) go to a staging copy of the
//     region in LDS at their final byte offset, then the region is written to HBM with
//     16-byte stores.
// Layout citations: [LBRS] "State bit allocation", "Levels and storage".
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256, NCG = 16;
constexpr float kMagic = 12582912.0f;          // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

struct BaSmem {
    uint32_t reg[(DK * DV + 3 * DK) / 4 + 8];  // staged region (codes, Delta, meta)
    int order[DK];                             // physical row at sorted position
    int off[DK];                               // byte offset of each row's codes
    int width[DK];
    float alpha[DK];                           // a_i * Delta_i (old)
    float beta0[DK];                           // -n_i * a_i * Delta_i
    float kk[DK], qq[DK];
    float fn[DK];                              // f_i / n_i
    float red[4][2][DV];
    float w[DV];
    int hist[16];
    float qk;
};

// 8 codes of `B` bits starting at byte `boff` of the staged region, as integers.
template <int B>
__device__ __forceinline__ void unpack8(const BaSmem& sm, int boff, uint32_t code[8]) {
    const uint8_t* bytes = reinterpret_cast<const uint8_t*>(sm.reg);
    if constexpr (B == 2) {
        const uint32_t v = *reinterpret_cast<const uint16_t*>(bytes + boff);
#pragma unroll
        for (int c = 0; c < 8; ++c) code[c] = (v >> (2 * c)) & 3u;
    } else if constexpr (B == 4) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(bytes + boff);
#pragma unroll
        for (int c = 0; c < 8; ++c) code[c] = (v >> (4 * c)) & 15u;
    } else if constexpr (B == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(bytes + boff);
#pragma unroll
        for (int c = 0; c < 4; ++c) code[c] = (v.x >> (8 * c)) & 255u;
#pragma unroll
        for (int c = 0; c < 4; ++c) code[4 + c] = (v.y >> (8 * c)) & 255u;
    } else {
        // B bytes at an arbitrary byte offset: three aligned words, funnel-shifted
        const int wi = boff >> 2, sh = (boff & 3) * 8;
        const uint32_t w0 = sm.reg[wi], w1 = sm.reg[wi + 1], w2 = sm.reg[wi + 2];
        const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);
        const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, sh);
        constexpr uint32_t M = (1u << B) - 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int p = c * B;
            if (p + B <= 32) code[c] = (lo >> p) & M;
            else if (p >= 32) code[c] = (hi >> (p - 32)) & M;
            else code[c] = __builtin_amdgcn_alignbit(hi, lo, p) & M;
        }
    }
}

// Round 8 values on the row grid and write the packed B-bit codes (b bytes) at byte
// `boff` of the staging copy.
template <int B>
__device__ __forceinline__ void pack8_store(BaSmem& sm, int boff, const float x[8], float inv, int n) {
    const float magic = kMagic + float(n);
    const float hi_f = kMagic + float(2 * n);
    uint32_t y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float t = __builtin_fmaf(x[c], inv, magic);       // kMagic + n + rne(x / Delta)
        y[c] = __float_as_uint(__builtin_amdgcn_fmed3f(t, kMagic, hi_f));
    }
    // shift-add the biased patterns, then remove the constant bias once per word
    uint32_t w0 = 0, w1 = 0;
    uint32_t g0 = 0, g1 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int p = c * B;
        if (p + B <= 32) {
            w0 += y[c] << p;
            g0 += kMagicBits << p;
        } else if (p >= 32) {
            w1 += y[c] << (p - 32);
            g1 += kMagicBits << (p - 32);
        } else {
            const uint32_t code = y[c] - kMagicBits;
            w0 += code << p;
            w1 += code >> (32 - p);
        }
    }
    w0 -= g0;
    w1 -= g1;
    uint8_t* bytes = reinterpret_cast<uint8_t*>(sm.reg);
    if constexpr (B == 2) {
        *reinterpret_cast<uint16_t*>(bytes + boff) = uint16_t(w0);
    } else if constexpr (B == 4) {
        *reinterpret_cast<uint32_t*>(bytes + boff) = w0;
    } else if constexpr (B == 8) {
        *reinterpret_cast<uint2*>(bytes + boff) = make_uint2(w0, w1);
    } else if constexpr (B == 6) {
        uint16_t* h = reinterpret_cast<uint16_t*>(bytes + boff);   // 2-byte aligned
        h[0] = uint16_t(w0);
        h[1] = uint16_t(w0 >> 16);
        h[2] = uint16_t(w1);
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i) bytes[boff + i] = uint8_t(i < 4 ? (w0 >> (8 * i)) : (w1 >> (8 * (i - 4))));
    }
}

// Row maximum over the 16 lanes of a row group (DPP inside a row of 16 lanes).
__device__ __forceinline__ float rowmax16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // xor 1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // xor 2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false))); // half mirror
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false))); // mirror
    return v;
}

// One workgroup per head state. The region and the per-row inputs are fetched into
// registers first, then written to LDS.
template <int MODE>
__global__ void __launch_bounds__(NT) bitalloc_step_kernel(const KArgs A, int num_heads) {
    __shared__ BaSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = lane >> 4;            // rq: row within the wave's quad
    const int code_bytes = DK * DV * A.bbar / 8;
    const int total = code_bytes + 3 * DK;
    const int nvec = (total + 15) / 16;

    uint4 pf0 = make_uint4(0, 0, 0, 0), pf1 = pf0, pf2 = pf0;
    float pk = 0.f, pq = 0.f, ps = 0.f, pv = 0.f;
#define WB_PREFETCH(hd)                                                                         \
    do {                                                                                        \
        const uint4* src_ = reinterpret_cast<const uint4*>(A.state + (size_t)(hd) * A.region_stride); \
        if (tid < nvec) pf0 = src_[tid];                                                        \
        if (tid + NT < nvec) pf1 = src_[tid + NT];                                              \
        if (tid + 2 * NT < nvec) pf2 = src_[tid + 2 * NT];                                      \
        if (tid < DK) {                                                                         \
            const size_t vb_ = (size_t)(hd) * DK + tid;                                         \
            pk = A.k[vb_];                                                                      \
            pq = A.q[vb_];                                                                      \
            ps = A.s_per_row ? A.s[vb_] : A.s[hd];                                              \
            pv = A.v[(size_t)(hd) * DV + tid];                                                  \
        }                                                                                       \
    } while (0)
    int head = blockIdx.x;
    WB_PREFETCH(head);

    {
        uint8_t* region = A.state + (size_t)head * A.region_stride;
        __syncthreads();                              // previous head is out of LDS
        {
            uint4* dst = reinterpret_cast<uint4*>(sm.reg);
            if (tid < nvec) dst[tid] = pf0;
            if (tid + NT < nvec) dst[tid + NT] = pf1;
            if (tid + 2 * NT < nvec) dst[tid + 2 * NT] = pf2;
        }
        if (tid < 16) sm.hist[tid] = 0;
        const float kv_row = pk, qv_row = pq, s_row = ps, v_col = pv;
        const float beta = A.beta[head];
        __syncthreads();

        // ---- per-row constants (threads 0..127 own row = tid) -----------------------
        const uint8_t* bytes = reinterpret_cast<const uint8_t*>(sm.reg);
        int my_w = 0;
        if (tid < DK) {
            const int r = tid;
            const int meta = bytes[code_bytes + 2 * DK + r];
            my_w = (meta & 7) + 1;
            const int fit = meta >> 4;
            const int n = (1 << (my_w - 1)) - 1;
            const float dl = f16_bits_to_f32(uint32_t(bytes[code_bytes + 2 * r]) |
                                             (uint32_t(bytes[code_bytes + 2 * r + 1]) << 8));
            const float a = expf(-s_row);
            sm.width[r] = my_w;
            sm.alpha[r] = a * dl;
            sm.beta0[r] = -float(n) * (a * dl);
            sm.kk[r] = kv_row;
            sm.qq[r] = qv_row;
            sm.fn[r] = float((0.25 + double(fit) / 20.0) / double(n));
            atomicAdd(&sm.hist[my_w], 1);
            int incl = my_w * (DV / 8);
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            sm.off[r] = incl - my_w * (DV / 8);
            float pqk = qv_row * kv_row;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) pqk += __shfl_xor(pqk, d, 64);
            if (lane == 63) sm.red[wave][0][0] = float(incl);
            if (lane == 0) sm.red[wave][1][0] = pqk;
        }
        __syncthreads();
        if (tid < DK) {
            const int r = tid;
            if (wave == 1) sm.off[r] += int(sm.red[0][0][0]);
            int base = 0;
            for (int v = 2; v < my_w; ++v) base += sm.hist[v];
            int rank = 0;
            for (int v = 2; v <= 8; ++v) {
                const unsigned long long m = __ballot(my_w == v);
                if (my_w == v) rank = __popcll(m & ((1ull << lane) - 1));
            }
            if (wave == 1) {
                int c0 = 0;
                for (int rr = 0; rr < 64; ++rr) c0 += (sm.width[rr] == my_w) ? 1 : 0;
                rank += c0;
            }
            sm.order[base + rank] = r;
            if (tid == 0) sm.qk = sm.red[0][1][0] + sm.red[1][1][0];
        }
        __syncthreads();

        // ---- dequantize the lane's 8 rows x 8 columns; u, p partial sums ------------
        // (the sorted-position base is re-materialised every head: keeping per-m LDS
        // addresses live across the head loop costs registers the tile needs)
        int pos0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(pos0));
        pos0 += 4 * wave + rq;
        float x[8][8];
        float up[8], pp[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            up[c] = 0.f;
            pp[c] = 0.f;
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int r = sm.order[16 * m + pos0];
            const int bw = sm.width[r];
            const int boff = sm.off[r] + cg * bw;
            uint32_t code[8];
            switch (bw) {
                case 2: unpack8<2>(sm, boff, code); break;
                case 3: unpack8<3>(sm, boff, code); break;
                case 4: unpack8<4>(sm, boff, code); break;
                case 5: unpack8<5>(sm, boff, code); break;
                case 6: unpack8<6>(sm, boff, code); break;
                case 7: unpack8<7>(sm, boff, code); break;
                default: unpack8<8>(sm, boff, code); break;
            }
            const float al = sm.alpha[r], b0 = sm.beta0[r], kv = sm.kk[r], qv = sm.qq[r];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                x[m][c] = __builtin_fmaf(float(code[c]), al, b0);
                up[c] = __builtin_fmaf(kv, x[m][c], up[c]);
                pp[c] = __builtin_fmaf(qv, x[m][c], pp[c]);
            }
            __builtin_amdgcn_sched_barrier(0);       // keep one row's temporaries live at a time
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            up[c] += __shfl_xor(up[c], 16, 64);
            up[c] += __shfl_xor(up[c], 32, 64);
            pp[c] += __shfl_xor(pp[c], 16, 64);
            pp[c] += __shfl_xor(pp[c], 32, 64);
        }
        if (rq == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                sm.red[wave][0][8 * cg + c] = up[c];
                sm.red[wave][1][8 * cg + c] = pp[c];
            }
        }
        __syncthreads();

        // ---- w = beta (v - u), o = p + (q . k) w ---------------------------------------
        if (tid < DV) {
            const int j = tid;
            const float u = (sm.red[0][0][j] + sm.red[1][0][j]) + (sm.red[2][0][j] + sm.red[3][0][j]);
            const float p = (sm.red[0][1][j] + sm.red[1][1][j]) + (sm.red[2][1][j] + sm.red[3][1][j]);
            const float wj = beta * (v_col - u);
            sm.w[j] = wj;
            A.o[(size_t)head * DV + j] = __builtin_fmaf(sm.qk, wj, p);
        }
        __syncthreads();

        // ---- update, row maxima ---------------------------------------------------------
        float wv[8];
        {
            const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[8 * cg]);
            const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[8 * cg + 4]);
            wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
            wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
        }
        float R[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float kv = sm.kk[sm.order[16 * m + pos0]];
#pragma unroll
            for (int c = 0; c < 8; ++c) x[m][c] = __builtin_fmaf(kv, wv[c], x[m][c]);
            float mx = fmaxf(fmaxf(fabsf(x[m][0]), fabsf(x[m][1])), fabsf(x[m][2]));
            mx = fmaxf(fmaxf(mx, fabsf(x[m][3])), fabsf(x[m][4]));
            mx = fmaxf(fmaxf(mx, fabsf(x[m][5])), fabsf(x[m][6]));
            R[m] = rowmax16(fmaxf(mx, fabsf(x[m][7])));
        }

        // ---- round and pack into the staging copy (every code byte is rewritten) --------
        uint16_t* dout = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(sm.reg) + code_bytes);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int r = sm.order[16 * m + pos0];
            const int bw = sm.width[r];
            const int n = (1 << (bw - 1)) - 1;
            const uint16_t dbits = f32_to_f16_bits(R[m] * sm.fn[r]);
            const float dl = f16_bits_to_f32(dbits);
            const float inv = dl > 0.f ? __builtin_amdgcn_rcpf(dl) : 0.f;
            const int boff = sm.off[r] + cg * bw;
            if (cg == 0) dout[r] = dbits;
            switch (bw) {
                case 2: pack8_store<2>(sm, boff, x[m], inv, n); break;
                case 3: pack8_store<3>(sm, boff, x[m], inv, n); break;
                case 4: pack8_store<4>(sm, boff, x[m], inv, n); break;
                case 5: pack8_store<5>(sm, boff, x[m], inv, n); break;
                case 6: pack8_store<6>(sm, boff, x[m], inv, n); break;
                case 7: pack8_store<7>(sm, boff, x[m], inv, n); break;
                default: pack8_store<8>(sm, boff, x[m], inv, n); break;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        {
            const int out_vec = (code_bytes + 2 * DK) / 16;
            uint4* dst = reinterpret_cast<uint4*>(region);
            const uint4* src = reinterpret_cast<const uint4*>(sm.reg);
            for (int i = tid; i < out_vec; i += NT) dst[i] = src[i];
        }
    }
#undef WB_PREFETCH
}

}  // namespace

hipError_t launch_bitalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream) {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    const int heads = d.B * d.H;
    hipLaunchKernelGGL(bitalloc_step_kernel<WB_RTN>, dim3(heads), dim3(NT), 0, stream, a, heads);
    return hipGetLastError();
}

}  // namespace wb
