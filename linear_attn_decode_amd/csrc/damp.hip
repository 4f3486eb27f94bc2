// DAMP row selection from sampled states (offline, once per layer): one workgroup per
// head walks the N samples.
//
// [DAMP] "Risk scoring and selection": E_u is the mean squared quantization-error
// energy of row u under the low-precision mapping (Hadamard rotation along dv, then
// per-block asymmetric affine INT8, nearest rounding); with constant decay the
// geometric-mean retention is a_u = e^{-s_u}; P_u = 1 / max(1 - a_u^2, tau);
// C_u = E_u P_u; the k_hi highest-cost rows are protected. [DAMP] "Implementation":
// the permutation lists the protected rows contiguously (ascending), then the others
// (ascending); ties in C go to the lower row index.
//
// The error energy is accumulated in the rotated domain, which equals the original
// domain's because the transform is orthonormal.
#include "wb_device.hpp"
#include "wb_kernels.hpp"

namespace wb {
namespace {

constexpr int DK = 128, DV = 128, NT = 256, NCG = 16, RS = 16;
constexpr double kInvSqrt128d = 0.08838834764831844055;

__device__ __forceinline__ void row_wht(double v[8], int cg) {
#pragma unroll
    for (int span = 1; span < 8; span <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & span) == 0) {
                const double a = v[i], b = v[i + span];
                v[i] = a + b;
                v[i + span] = a - b;
            }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double o = __shfl_xor(v[i], d, 64);
            v[i] = (cg & d) ? (o - v[i]) : (v[i] + o);
        }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= kInvSqrt128d;
}

__global__ void __launch_bounds__(NT) damp_kernel(const DampArgs A) {
    __shared__ double cost[DK];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    const int LB = A.block / 8;
    double E[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int n = 0; n < A.N; ++n) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int row = rg + RS * m;
            const float* src = A.samples + (((size_t)n * A.H + h) * DK + row) * DV + 8 * cg;
            const float4 v0 = reinterpret_cast<const float4*>(src)[0];
            const float4 v1 = reinterpret_cast<const float4*>(src)[1];
            double y[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            row_wht(y, cg);
            double mn = y[0], mx = y[0];
#pragma unroll
            for (int c = 1; c < 8; ++c) {
                mn = fmin(mn, y[c]);
                mx = fmax(mx, y[c]);
            }
            for (int d = 1; d < LB; d <<= 1) {
                mn = fmin(mn, __shfl_xor(mn, d, 64));
                mx = fmax(mx, __shfl_xor(mx, d, 64));
            }
            const double scale = double(f16_bits_to_f32(f64_to_f16_bits(fmax(mx - mn, 0.0) / 255.0)));
            const double zero = double(f16_bits_to_f32(f64_to_f16_bits(mn)));
            double e = 0.0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                double kap = 0.0;
                if (scale != 0.0) kap = fmin(fmax(rint((y[c] - zero) / scale), 0.0), 255.0);
                const double r = y[c] - (zero + kap * scale);
                e += r * r;
            }
            E[m] += e;
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int d = 1; d < NCG; d <<= 1) E[m] += __shfl_xor(E[m], d, 64);
        if (cg == 0) {
            const int row = rg + RS * m;
            const double a = exp(-double(A.s[(size_t)h * DK + row]));
            const double P = 1.0 / fmax(1.0 - a * a, double(A.tau));
            cost[row] = (E[m] / double(A.N)) * P;
        }
    }
    __syncthreads();
    if (tid < DK) {
        const int u = tid;
        const double cu = cost[u];
        int rank = 0;
        for (int v = 0; v < DK; ++v) {
            const double cv = cost[v];
            rank += (cv > cu || (cv == cu && v < u)) ? 1 : 0;
        }
        const bool sel = rank < A.k_hi;
        int pos = 0;
        for (int v = 0; v < u; ++v) {
            const double cv = cost[v];
            int rv = 0;
            for (int w = 0; w < DK; ++w) {
                const double cw = cost[w];
                rv += (cw > cv || (cw == cv && w < v)) ? 1 : 0;
            }
            pos += ((rv < A.k_hi) == sel) ? 1 : 0;
        }
        A.perm[(size_t)h * DK + (sel ? pos : A.k_hi + pos)] = uint8_t(u);
        if (A.cost) A.cost[(size_t)h * DK + u] = float(cu);
    }
}

}  // namespace

hipError_t launch_damp_select(const DampArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(damp_kernel, dim3(a.H), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wb
