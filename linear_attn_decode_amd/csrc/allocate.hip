// Decay-aware per-row bit allocation pass (BITALLOC layout), one workgroup per head.
//
// [LBRS] "Approximate erasure rate", "Range normalization", "State bit allocation",
// "Levels and storage"; [LBRS-x] (cost c = Gamma-hat * R~^2 and the width rule):
//   R_i   = max_j |S_ij| of the stored state;  R~_i = R_i / RMS_j R_j (one head);
//   Gamma = 1 / expm1(2 (s_i + r_i));  c_i = max(Gamma R~_i^2, 1e-300);
//   b*_i  = bbar + 0.5 log2(c_i / GM(c));  b_i = clip(rint(b*_i), bmin, bmax), then one
//   bit at a time: while short, +1 to the largest (3/4) c 2^{-2b} among b < bmax; while
//   over, -1 to the smallest 3 c 2^{-2b} among b > bmin; ties to the lower row;
//   all R_i = 0 keeps every row at bbar;
//   fit: f_k = 1/4 + k/20, Delta_k = f16(f_k R_i / n_i), the smallest squared rounding
//   error wins, ties to the larger f;
//   repack: the stored values rounded to nearest on the new grid, new prefix offsets.
// Everything that decides a width or a fit index runs in float64; the pass is rare
// (every 64 tokens in the decay-aware decode study), so it favours exactness.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256, NCG = 16, RS = 16;

struct AllocSmem {
    uint32_t reg[(DK * DV + 3 * DK) / 4 + 4];
    int width[DK], fit[DK], off[DK], newoff[DK];
    float delta[DK];
    double R[DK], c[DK];
    int newwidth[DK];
    int newfit[DK];
    uint16_t newdelta[DK];
};

__device__ __forceinline__ void argbest(double& val, int& idx, bool want_max) {
    // wave-wide arg-max (or arg-min) with ties to the lower index
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double ov = __shfl_xor(val, d, 64);
        const int oi = __shfl_xor(idx, d, 64);
        const bool better = want_max ? (ov > val || (ov == val && oi < idx)) : (ov < val || (ov == val && oi < idx));
        if (better) {
            val = ov;
            idx = oi;
        }
    }
}

__global__ void __launch_bounds__(NT) allocate_kernel(const AllocArgs A) {
    __shared__ AllocSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int head = blockIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    uint8_t* region = A.state + (size_t)head * A.region_stride;
    const int code_bytes = DK * DV * A.bbar / 8;
    const int total = code_bytes + 3 * DK;

    for (int i = tid; i * 16 < total; i += NT)
        reinterpret_cast<uint4*>(sm.reg)[i] = reinterpret_cast<const uint4*>(region)[i];
    __syncthreads();
    const uint8_t* bytes = reinterpret_cast<const uint8_t*>(sm.reg);
    if (wave == 0) {
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
    }
    __syncthreads();

    // stored values (exact in float32: |kappa| <= 127 times a float16 Delta)
    double x[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int row = rg + RS * m;
        const int bw = sm.width[row];
        const int n = (1 << (bw - 1)) - 1;
        const int off = sm.off[row] + cg * bw;
        const int wi = off >> 2, sh = (off & 3) * 8;
        uint64_t fld = (uint64_t(sm.reg[wi]) | (uint64_t(sm.reg[wi + 1]) << 32)) >> sh;
        if (sh) fld |= uint64_t(sm.reg[wi + 2]) << (64 - sh);
        const float dl = sm.delta[row];
        double R = 0.0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int kap = int((fld >> (c * bw)) & ((1ull << bw) - 1)) - n;
            x[m][c] = double(float(kap) * dl);
            R = fmax(R, fabs(x[m][c]));
        }
#pragma unroll
        for (int d = 1; d < NCG; d <<= 1) R = fmax(R, __shfl_xor(R, d, 64));
        if (cg == 0) sm.R[row] = R;
    }
    __syncthreads();

    // widths (one wavefront; lane l owns rows 2l and 2l+1)
    if (wave == 0) {
        const int r0 = 2 * lane, r1 = r0 + 1;
        const double R0 = sm.R[r0], R1 = sm.R[r1];
        double sq = R0 * R0 + R1 * R1;
        double anyR = fmax(R0, R1);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            sq += __shfl_xor(sq, d, 64);
            anyR = fmax(anyR, __shfl_xor(anyR, d, 64));
        }
        int b0 = A.bbar, b1 = A.bbar;
        double c0 = 0.0, c1 = 0.0;
        if (anyR > 0.0) {
            const double rms = sqrt(sq / double(DK));
            const size_t base = (size_t)head * DK;
            const double s0 = A.s[base + r0], s1 = A.s[base + r1];
            const double q0 = A.r ? double(A.r[base + r0]) : double(A.r_default);
            const double q1 = A.r ? double(A.r[base + r1]) : double(A.r_default);
            const double g0 = 1.0 / expm1(2.0 * (s0 + q0));
            const double g1 = 1.0 / expm1(2.0 * (s1 + q1));
            const double rt0 = R0 / rms, rt1 = R1 / rms;
            c0 = fmax(g0 * (rt0 * rt0), 1e-300);
            c1 = fmax(g1 * (rt1 * rt1), 1e-300);
            double lsum = log(c0) + log(c1);
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) lsum += __shfl_xor(lsum, d, 64);
            const double gm = exp(lsum / double(DK));
            const double bs0 = double(A.bbar) + 0.5 * log2(c0 / gm);
            const double bs1 = double(A.bbar) + 0.5 * log2(c1 / gm);
            b0 = int(fmin(fmax(rint(bs0), double(A.bmin)), double(A.bmax)));
            b1 = int(fmin(fmax(rint(bs1), double(A.bmin)), double(A.bmax)));
            const int target = A.bbar * DK;
            for (int iter = 0; iter < 4 * DK * 8; ++iter) {   // each pass moves one bit toward the budget
                int tot = b0 + b1;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) tot += __shfl_xor(tot, d, 64);
                if (tot == target) break;
                const bool grow = tot < target;
                double v0, v1;
                if (grow) {
                    v0 = b0 < A.bmax ? (0.75 * c0) * exp2(-2.0 * b0) : -INFINITY;
                    v1 = b1 < A.bmax ? (0.75 * c1) * exp2(-2.0 * b1) : -INFINITY;
                } else {
                    v0 = b0 > A.bmin ? (3.0 * c0) * exp2(-2.0 * b0) : INFINITY;
                    v1 = b1 > A.bmin ? (3.0 * c1) * exp2(-2.0 * b1) : INFINITY;
                }
                double bv;
                int bi;
                if (grow) {
                    bv = (v1 > v0) ? v1 : v0;
                    bi = (v1 > v0) ? r1 : r0;
                } else {
                    bv = (v1 < v0) ? v1 : v0;
                    bi = (v1 < v0) ? r1 : r0;
                }
                argbest(bv, bi, grow);
                if (bi == r0) b0 += grow ? 1 : -1;
                if (bi == r1) b1 += grow ? 1 : -1;
            }
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
    }
    __syncthreads();

    // clipping fit and repack
    for (int i = tid; i < code_bytes / 4; i += NT) sm.reg[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int row = rg + RS * m;
        const int bw = sm.newwidth[row];
        const int n = (1 << (bw - 1)) - 1;
        const double R = sm.R[row];
        double err[16];
#pragma unroll
        for (int kf = 0; kf < 16; ++kf) {
            const double d = double(__half2float(__ushort_as_half(f64_to_f16_bits((0.25 + kf / 20.0) * R / n))));
            double e = 0.0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                double kap = 0.0;
                if (d != 0.0) kap = fmin(fmax(rint(x[m][c] / d), double(-n)), double(n));
                const double r = x[m][c] - d * kap;
                e += r * r;
            }
#pragma unroll
            for (int dd = 1; dd < NCG; dd <<= 1) e += __shfl_xor(e, dd, 64);
            err[kf] = e;
        }
        int best = 15;
#pragma unroll
        for (int kf = 14; kf >= 0; --kf)
            if (err[kf] < err[best]) best = kf;
        const uint16_t dbits = f64_to_f16_bits((0.25 + best / 20.0) * R / n);
        const double d = double(f16_bits_to_f32(dbits));
        uint64_t fld = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            double kap = 0.0;
            if (d != 0.0) kap = fmin(fmax(rint(x[m][c] / d), double(-n)), double(n));
            fld |= uint64_t(int(kap) + n) << (c * bw);
        }
        const int off = sm.newoff[row] + cg * bw;
        const int wi = off >> 2, sh = (off & 3) * 8;
        const uint64_t lo = fld << sh;
        atomicOr(&sm.reg[wi], uint32_t(lo));
        atomicOr(&sm.reg[wi + 1], uint32_t(lo >> 32));
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

}  // namespace

hipError_t launch_allocate_bits(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(allocate_kernel, dim3(d.B * d.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wb
