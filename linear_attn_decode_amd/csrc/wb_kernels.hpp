// Kernel argument blocks and launch entry points of the write-back kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wbstate.h"

namespace wb {

enum Op : int { OP_STEP = 0, OP_IMPORT = 1, OP_EXPORT = 2 };

struct KArgs {
    uint8_t* state = nullptr;         // first region
    float* side = nullptr;            // error-feedback residuals [B*H][dk][dv]
    const uint8_t* perm = nullptr;    // [H][dk] (MIXED)
    const float* q = nullptr;
    const float* k = nullptr;
    const float* v = nullptr;
    const float* beta = nullptr;
    const float* s = nullptr;
    float* o = nullptr;
    const float* S_in = nullptr;      // import: [B*H][dk][dv] logical order
    float* S_out = nullptr;           // export
    uint64_t t = 0;
    uint64_t seed = 0;
    uint64_t region_stride = 0;
    int H = 1;
    int s_per_row = 1;
    int bits = 4;
    int block = 32;
    int k_hi = 0;
    int bbar = 4;
    int bmin = 2;                     // BITALLOC smallest row width
    int mem_bits = 0;                 // k of direction / residual memory
    int code_cap = 0;                 // BITALLOC code-area bytes of a head (meta follows)
    int layer = 0;                    // BITALLOC layer budget: the used code bytes vary per head
    int head_unit = 0;                // HEADALLOC (run by the BITALLOC kernels): one width, group scales
    int int_bits = 8;                 // HAD_INT8 / MIXED integer tier: 8 or 4
    uint32_t* activity = nullptr;     // [B*H][8] write-activity counters (UNIFORM) or null
    uint8_t* votes = nullptr;         // [B*H][DK][DV] vote state, with `activity`
    float* est = nullptr;             // [B*H][2 DK + 4] online estimators (BITALLOC) or null
};

// One launch of the decode / import / export kernel for every head of the layout.
hipError_t launch_wb(const wb_layout_desc& d, int op, const KArgs& a, hipStream_t stream);

// Decode step of the BITALLOC layout with round-to-nearest (the tuned kernel), for the
// layouts bitalloc_step_supported() accepts (either budget, one-bit rows included).
bool bitalloc_step_supported(const wb_layout_desc& d);
hipError_t launch_bitalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream);

// Decode step of the per-head allocation unit (HEADALLOC) with round-to-nearest or
// stochastic rounding.
bool headalloc_step_supported(const wb_layout_desc& d);
hipError_t launch_headalloc_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream);

// Decode step of the Hadamard-rotated layouts under round-to-nearest, stochastic
// rounding or error feedback (the tuned kernel), for the shapes rot_step_supported()
// accepts.
bool rot_step_supported(const wb_layout_desc& d);
hipError_t launch_rot_step(const wb_layout_desc& d, const KArgs& a, hipStream_t stream);

// Fills `n` bytes at dst with the repeating `period`-byte pattern (period <= 16).
hipError_t launch_fill(void* dst, size_t n, const uint8_t* pattern, int period, hipStream_t stream);

// Writes the zero state of every BITALLOC region: codes of width bbar holding level 0
// (the `period`-byte pattern) on [0, code_bytes), Delta = 0 and the given meta byte
// after the code area of `cap` bytes.
hipError_t launch_init_bitalloc(uint8_t* state, uint64_t stride, int heads, int code_bytes, int cap,
                                const uint8_t* pattern, int period, int dk, uint8_t meta, hipStream_t stream);
// The same for HEADALLOC regions: codes, `groups` zero f16 scales, fit index 15 per
// group, the width byte.
hipError_t launch_init_headalloc(uint8_t* state, uint64_t stride, int heads, int code_bytes, int cap,
                                 const uint8_t* pattern, int period, int groups, uint8_t wbyte, hipStream_t stream);

struct AllocArgs {
    uint8_t* state = nullptr;
    const float* s = nullptr;         // [B*H][dk]
    const float* r = nullptr;         // [B*H][dk] or null
    float* est = nullptr;             // [B*H][2 dk + 4] online estimators, used when s is null
    int factor = 0;                   // WB_GAMMA_*
    int cadence = 1;                  // C of the persistence factor
    // decode step whose write-back allocates (launch_step_allocate): the token's inputs
    const float *q = nullptr, *k = nullptr, *v = nullptr, *beta = nullptr, *sd = nullptr;
    float* o = nullptr;
    uint64_t t = 0;                   // the token index (stochastic rounding draws)
    uint64_t seed = 0;
    int s_per_row = 1;
    uint64_t region_stride = 0;
    float r_default = 0.f;
    int bbar = 4, bmin = 2, bmax = 8;
    // layer-wise budget: code-area bytes and the workspace of costs and widths
    int code_cap = 0;
    int H = 1;
    int rows_per_seq = 0;             // allocation units of a sequence: H*dk rows, or H heads
    double* ws_c = nullptr;           // [B*rows_per_seq]
    uint8_t* ws_w = nullptr;          // [B*rows_per_seq]
};
hipError_t launch_allocate_bits(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream);
hipError_t launch_step_allocate(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream);
// layer-wise budget: costs per head, widths per sequence, then fits and repack per head
hipError_t launch_allocate_layer(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream);
// per-head unit (HEADALLOC): head costs, widths per sequence, then group fits and repack
hipError_t launch_allocate_heads(const wb_layout_desc& d, const AllocArgs& a, hipStream_t stream);

struct DampArgs {
    const float* samples = nullptr;   // [N][H][dk][dv]
    const float* s = nullptr;         // [H][dk]
    float* cost = nullptr;            // [H][dk] or null
    uint8_t* perm = nullptr;          // [H][dk]
    int N = 0, H = 0, block = 32, k_hi = 16;
    float tau = 0.01f;
};
hipError_t launch_damp_select(const DampArgs& a, hipStream_t stream);

struct PrefillArgs {
    KArgs base;                       // state, side, perm, seed, region_stride, H, ...
    const uint16_t* q = nullptr;      // [B][T][H][dk] bf16
    const uint16_t* k = nullptr;
    const uint16_t* v = nullptr;
    const float* beta = nullptr;      // [B][T][H]
    const float* s = nullptr;         // [B][T][H][dk] or [B][T][H]
    float* o = nullptr;               // [B][T][H][dv]
    int T = 0, chunk = 64, C = 8;
    uint64_t t0 = 0;
};
hipError_t launch_prefill(const wb_layout_desc& d, const PrefillArgs& a, hipStream_t stream);

}  // namespace wb
