// Host side of the C ABI (include/wbstate.h): descriptor validation, buffer sizing,
// handle management and kernel dispatch. No device memory is allocated here; every
// device buffer belongs to the caller.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "wb_kernels.hpp"
#include "wbstate.h"

struct wb_state {
    wb_layout_desc d;
    uint8_t* state;
    size_t state_bytes;
    float* side;
    size_t side_bytes;
    size_t region_stride;
    size_t regions_bytes;
    uint8_t* perm_dev;     // inside the state buffer (MIXED), else null
    uint32_t* activity;    // caller's write-activity counters (UNIFORM), or null
    uint8_t* votes;        // caller's per-element vote state, set with `activity`
    float* est;            // caller's online estimators (BITALLOC), or null
    uint8_t* scratch;      // device address of this GPU's `scratch` array, or null
};

namespace {

// Scratch of state_allocate_bits_static: the workspace the allocation passes of the
// layer-wise budget and the per-head unit otherwise keep after the regions (a float64
// cost and a uint8 width per row of the layer: 9 bytes per row). Each GPU the library
// runs on holds its own copy until the process ends. Nothing in it has to start at
// zero: every pass writes each row's cost and width before reading them.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address on each GPU, looked up once per device with that device
// current. In host code `scratch` names a host-side stand-in, never the device memory.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint8_t* scratch_addr[kMaxDevices] = {};

uint8_t* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_addr[dev] = static_cast<uint8_t*>(p);
    }
    return scratch_addr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// BITALLOC code-area bytes of one head: exactly the budget (per-head budget) or room
// for every row at bmax (layer budget)
size_t code_capacity(const wb_layout_desc& d) {
    const bool room = d.budget == WB_BUDGET_LAYER || d.kind == WB_HEADALLOC;
    return size_t(d.dk) * d.dv * size_t(room ? d.bmax : d.bbar) / 8;
}

// width of the integer tier of the Hadamard layouts
size_t int_bits(const wb_layout_desc& d) { return d.int_bits == 4 ? 4 : 8; }

size_t region_size(const wb_layout_desc& d) {
    const size_t dk = d.dk, dv = d.dv;
    switch (d.kind) {
        case WB_FP32: return 4 * dk * dv;
        case WB_UNIFORM: return dk * dv * size_t(d.bits) / 8;
        case WB_HAD_INT8: return dk * dv * int_bits(d) / 8 + dk * (dv / d.block) * 4;
        case WB_MIXED: {
            const size_t qr = dk - size_t(d.k_hi);
            return size_t(d.k_hi) * dv * 2 + qr * dv * int_bits(d) / 8 + qr * (dv / d.block) * 4;
        }
        case WB_HEADALLOC: return code_capacity(d) + 3 * (dk / 32) * dv + 16;
        default: return code_capacity(d) + 3 * dk;
    }
}

// workspace of the layer-wise allocation, after the regions: float64 costs and u8
// widths of every row
size_t layer_ws_size(const wb_layout_desc& d) {
    if (d.kind == WB_HEADALLOC) return round256(size_t(d.B) * d.H * 9);      // one "row" per head
    if (d.kind != WB_BITALLOC || d.budget != WB_BUDGET_LAYER) return 0;
    return round256(size_t(d.B) * d.H * d.dk * 9);
}

int validate(const wb_layout_desc* d) {
    if (!d) return WB_EINVAL;
    if (d->kind < WB_FP32 || d->kind > WB_HEADALLOC) return WB_EINVAL;
    if (d->mode < WB_RTN || d->mode > WB_RESQ) return WB_EINVAL;
    if (d->decay != WB_DECAY_PER_HEAD && d->decay != WB_DECAY_PER_ROW) return WB_EINVAL;
    const bool memory_rule = d->mode == WB_DIR || d->mode == WB_RESQ;
    if (memory_rule ? (d->mem_bits < 1 || d->mem_bits > 8) : d->mem_bits != 0) return WB_EINVAL;
    if (memory_rule && d->kind != WB_UNIFORM) return WB_EUNSUPPORTED;
    if (d->B < 1 || d->H < 1) return WB_EINVAL;
    if ((int64_t)d->B * d->H > 0x7FFFFFFF) return WB_EUNSUPPORTED;
    const bool small = d->dk == 16 && d->dv == 16;
    const bool big = d->dk == 128 && d->dv == 128;
    if (d->kind == WB_FP32 || d->kind == WB_UNIFORM) {
        if (!small && !big) return WB_EUNSUPPORTED;
    } else if (!big) {
        return WB_EUNSUPPORTED;
    }
    if (d->kind == WB_UNIFORM && d->bits != 2 && d->bits != 4 && d->bits != 8) return WB_EUNSUPPORTED;
    if (d->kind == WB_HAD_INT8 || d->kind == WB_MIXED) {
        if (d->block != 32 && d->block != 64 && d->block != 128) return WB_EUNSUPPORTED;
        if (d->dv % d->block) return WB_EUNSUPPORTED;
    }
    if (d->kind == WB_MIXED) {
        const int rs = d->dk / 8;
        if (d->k_hi <= 0 || d->k_hi >= d->dk || d->k_hi % rs) return WB_EUNSUPPORTED;
    }
    if (d->kind == WB_BITALLOC || d->kind == WB_HEADALLOC) {
        // one-bit rows (bmin = 1) for the per-row unit only: a one-bit head is excluded
        const int floor = d->kind == WB_BITALLOC ? 1 : 2;
        if (d->bmin < floor || d->bmin > d->bbar || d->bbar > d->bmax || d->bmax > 8) return WB_EUNSUPPORTED;
    }
    if (d->kind == WB_HEADALLOC && d->H > 4096) return WB_EUNSUPPORTED;
    const bool hadamard = d->kind == WB_HAD_INT8 || d->kind == WB_MIXED;
    if (hadamard ? (d->int_bits != 0 && d->int_bits != 8 && d->int_bits != 4) : d->int_bits != 0) return WB_EINVAL;
    if (d->budget != WB_BUDGET_HEAD && d->budget != WB_BUDGET_LAYER) return WB_EINVAL;
    if (d->budget == WB_BUDGET_LAYER && (d->kind != WB_BITALLOC || d->H * d->dk > 4096)) return WB_EUNSUPPORTED;
    return WB_OK;
}

size_t side_size(const wb_layout_desc& d) {
    if ((d.mode != WB_EF && d.mode != WB_DIR && d.mode != WB_RESQ) || d.kind == WB_FP32) return 0;
    return size_t(d.B) * d.H * d.dk * d.dv * 4;
}

int hip_status(hipError_t e) { return e == hipSuccess ? WB_OK : WB_ELAUNCH; }

wb::KArgs base_args(const wb_state* st) {
    wb::KArgs a;
    a.state = st->state;
    a.side = st->side;
    a.perm = st->perm_dev;
    a.seed = st->d.seed;
    a.region_stride = st->region_stride;
    a.H = st->d.H;
    a.s_per_row = st->d.decay == WB_DECAY_PER_ROW;
    a.bits = st->d.bits;
    a.block = st->d.block;
    a.k_hi = st->d.k_hi;
    a.bbar = st->d.bbar;
    a.bmin = st->d.bmin;
    a.mem_bits = st->d.mem_bits;
    a.code_cap = int(code_capacity(st->d));
    a.int_bits = int(int_bits(st->d));
    a.head_unit = st->d.kind == WB_HEADALLOC;
    a.layer = (st->d.kind == WB_BITALLOC && st->d.budget == WB_BUDGET_LAYER) || a.head_unit;
    return a;
}

}  // namespace

extern "C" {

int state_bytes(const wb_layout_desc* d, size_t* state_bytes_out, size_t* side_bytes_out) {
    const int v = validate(d);
    if (v) return v;
    if (!state_bytes_out || !side_bytes_out) return WB_EINVAL;
    const size_t stride = round256(region_size(*d));
    size_t total = stride * size_t(d->B) * size_t(d->H);
    if (d->kind == WB_MIXED) total += round256(size_t(d->H) * d->dk);
    total += layer_ws_size(*d);
    *state_bytes_out = total;
    *side_bytes_out = side_size(*d);
    return WB_OK;
}

int state_alloc(const wb_layout_desc* d, void* dev_state, size_t state_bytes_in, void* dev_side,
                size_t side_bytes_in, const uint8_t* perm, void* stream, wb_state** out) {
    const int v = validate(d);
    if (v) return v;
    if (!out || !dev_state) return WB_EINVAL;
    size_t need = 0, need_side = 0;
    state_bytes(d, &need, &need_side);
    if (state_bytes_in < need) return WB_ESIZE;
    if (!aligned16(dev_state)) return WB_EALIGN;
    if (need_side) {
        if (!dev_side) return WB_EINVAL;
        if (side_bytes_in < need_side) return WB_ESIZE;
        if (!aligned16(dev_side)) return WB_EALIGN;
    }
    if (d->kind == WB_MIXED) {
        if (!perm) return WB_EINVAL;
        for (int h = 0; h < d->H; ++h) {
            uint8_t seen[256] = {0};
            for (int i = 0; i < d->dk; ++i) {
                const uint8_t p = perm[(size_t)h * d->dk + i];
                if (p >= d->dk || seen[p]) return WB_EINVAL;
                seen[p] = 1;
            }
        }
    }
    wb_state* st = new (std::nothrow) wb_state;
    if (!st) return WB_EINVAL;
    st->d = *d;
    st->state = static_cast<uint8_t*>(dev_state);
    st->state_bytes = state_bytes_in;
    st->side = need_side ? static_cast<float*>(dev_side) : nullptr;
    st->side_bytes = need_side ? side_bytes_in : 0;
    st->region_stride = round256(region_size(*d));
    st->regions_bytes = st->region_stride * size_t(d->B) * size_t(d->H);
    st->perm_dev = d->kind == WB_MIXED ? st->state + st->regions_bytes : nullptr;
    st->activity = nullptr;
    st->votes = nullptr;
    st->est = nullptr;
    // the static scratch of this device (null if the lookup failed: then only
    // state_allocate_bits_static refuses, with WB_ELAUNCH)
    st->scratch = scratch_for_current_device();
    hipStream_t s = static_cast<hipStream_t>(stream);

    // zero state: all layouts but BITALLOC encode S_0 = 0 as zero bytes
    const uint8_t zero = 0;
    hipError_t e = wb::launch_fill(st->state, st->regions_bytes, &zero, 1, s);
    if (e == hipSuccess && d->kind == WB_BITALLOC) {
        // every row at width bbar, level 0 stored as n = 2^(bbar-1) - 1, Delta = 0,
        // meta = (bbar - 1) | (15 << 4); a row of 8 fields is exactly bbar bytes
        const int bb = d->bbar;
        const uint64_t n = (1ull << (bb - 1)) - 1;
        uint64_t fields = 0;
        for (int c = 0; c < 8; ++c) fields |= n << (c * bb);
        uint8_t pat[8];
        for (int i = 0; i < bb; ++i) pat[i] = uint8_t(fields >> (8 * i));
        const int code_bytes = d->dk * d->dv * bb / 8;
        const uint8_t meta = uint8_t((bb - 1) | (15 << 4));
        e = wb::launch_init_bitalloc(st->state, st->region_stride, d->B * d->H, code_bytes, int(code_capacity(*d)),
                                     pat, bb, d->dk, meta, s);
    }
    if (e == hipSuccess && d->kind == WB_HEADALLOC) {
        // every element at width bbar holding level 0 (n), Delta = 0, fit indices 15
        const int bb = d->bbar;
        const uint64_t n = (1ull << (bb - 1)) - 1;
        uint64_t fields = 0;
        for (int c = 0; c < 8; ++c) fields |= n << (c * bb);
        uint8_t pat[8];
        for (int i = 0; i < bb; ++i) pat[i] = uint8_t(fields >> (8 * i));
        e = wb::launch_init_headalloc(st->state, st->region_stride, d->B * d->H, d->dk * d->dv * bb / 8,
                                      int(code_capacity(*d)), pat, bb, (d->dk / 32) * d->dv, uint8_t(bb - 1), s);
    }
    if (e == hipSuccess && st->side) e = wb::launch_fill(st->side, need_side, &zero, 1, s);
    if (e == hipSuccess && st->perm_dev) {
        e = hipMemcpyAsync(st->perm_dev, perm, size_t(d->H) * d->dk, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
    }
    if (e != hipSuccess) {
        delete st;
        return WB_ELAUNCH;
    }
    *out = st;
    return WB_OK;
}

int state_free(wb_state* st) {
    if (!st) return WB_EINVAL;
    delete st;
    return WB_OK;
}

int state_step_decode(wb_state* st, const float* q, const float* k, const float* v, const float* beta,
                      const float* s, float* o, uint64_t t, void* stream) {
    if (!st || !q || !k || !v || !beta || !s || !o) return WB_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(beta) || !aligned4(s))
        return WB_EALIGN;
    wb::KArgs a = base_args(st);
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.s = s;
    a.o = o;
    a.t = t;
    a.activity = st->activity;
    a.votes = st->votes;
    a.est = st->est;
    return hip_status(wb::launch_wb(st->d, wb::OP_STEP, a, static_cast<hipStream_t>(stream)));
}

int state_set_activity(wb_state* st, uint32_t* dev_counters, uint8_t* dev_votes) {
    if (!st) return WB_EINVAL;
    if (st->d.kind != WB_UNIFORM) return WB_EUNSUPPORTED;
    if ((dev_counters == nullptr) != (dev_votes == nullptr)) return WB_EINVAL;
    if (dev_counters && (!aligned16(dev_counters) || !aligned16(dev_votes))) return WB_EALIGN;
    st->activity = dev_counters;
    st->votes = dev_votes;
    return WB_OK;
}

int state_dequant(const wb_state* st, float* S, void* stream) {
    if (!st || !S) return WB_EINVAL;
    if (!aligned16(S)) return WB_EALIGN;
    wb::KArgs a = base_args(st);
    a.S_out = S;
    return hip_status(wb::launch_wb(st->d, wb::OP_EXPORT, a, static_cast<hipStream_t>(stream)));
}

int state_quantize(wb_state* st, const float* S, void* stream) {
    if (!st || !S) return WB_EINVAL;
    if (!aligned16(S)) return WB_EALIGN;
    wb::KArgs a = base_args(st);
    a.S_in = S;
    return hip_status(wb::launch_wb(st->d, wb::OP_IMPORT, a, static_cast<hipStream_t>(stream)));
}

int state_set_estimators(wb_state* st, float* dev_est) {
    if (!st) return WB_EINVAL;
    if (st->d.kind != WB_BITALLOC && st->d.kind != WB_HEADALLOC) return WB_EUNSUPPORTED;
    if (dev_est && !aligned16(dev_est)) return WB_EALIGN;
    st->est = dev_est;
    return WB_OK;
}

}  // extern "C"

namespace {

// The allocation pass; `ws` is the workspace of the layer-wise budget and the per-head
// unit: the state buffer's tail, or the static scratch (state_allocate_bits_static).
int allocate_bits(wb_state* st, const float* s, const float* r, int factor, int C, void* stream, uint8_t* ws) {
    wb::AllocArgs a;
    a.state = st->state;
    a.s = s;
    a.r = r;
    a.est = s ? nullptr : st->est;
    a.factor = factor;
    a.cadence = C;
    a.code_cap = int(code_capacity(st->d));
    a.region_stride = st->region_stride;
    a.r_default = float(1.0 / (3.0 * st->d.dk));
    a.bbar = st->d.bbar;
    a.bmin = st->d.bmin;
    a.bmax = st->d.bmax;
    if (st->d.kind == WB_HEADALLOC) {
        a.H = st->d.H;
        a.rows_per_seq = st->d.H;
        a.ws_c = reinterpret_cast<double*>(ws);
        a.ws_w = ws + size_t(st->d.B) * st->d.H * 8;
        return hip_status(wb::launch_allocate_heads(st->d, a, static_cast<hipStream_t>(stream)));
    }
    if (st->d.budget == WB_BUDGET_LAYER) {
        a.H = st->d.H;
        a.rows_per_seq = st->d.H * st->d.dk;
        a.ws_c = reinterpret_cast<double*>(ws);
        a.ws_w = ws + size_t(st->d.B) * st->d.H * st->d.dk * 8;
        return hip_status(wb::launch_allocate_layer(st->d, a, static_cast<hipStream_t>(stream)));
    }
    return hip_status(wb::launch_allocate_bits(st->d, a, static_cast<hipStream_t>(stream)));
}

int allocate_bits_check(const wb_state* st, const float* s, const float* r, int factor, int C) {
    if (!st) return WB_EINVAL;
    if (st->d.kind != WB_BITALLOC && st->d.kind != WB_HEADALLOC) return WB_EUNSUPPORTED;
    if (factor < WB_GAMMA_ERASURE || factor > WB_GAMMA_HC || C < 1) return WB_EINVAL;
    if (!s && (r || !st->est)) return WB_EINVAL;
    if ((s && !aligned4(s)) || (r && !aligned4(r))) return WB_EALIGN;
    return WB_OK;
}

}  // namespace

extern "C" {

int state_allocate_bits(wb_state* st, const float* s, const float* r, int factor, int C, void* stream) {
    const int v = allocate_bits_check(st, s, r, factor, C);
    if (v) return v;
    return allocate_bits(st, s, r, factor, C, stream, st->state + st->regions_bytes);
}

int state_allocate_bits_static(wb_state* st, const float* s, const float* r, int factor, int C, void* stream) {
    const int v = allocate_bits_check(st, s, r, factor, C);
    if (v) return v;
    // the same bytes the state's own workspace holds, which must fit the static array
    if (layer_ws_size(st->d) > kScratchBytes) return WB_ESCRATCH;
    if (!st->scratch) return WB_ELAUNCH;
    return allocate_bits(st, s, r, factor, C, stream, st->scratch);
}

int state_step_decode_alloc(wb_state* st, const float* q, const float* k, const float* v, const float* beta,
                            const float* s, float* o, uint64_t t, int factor, int C, void* stream) {
    if (!st || !q || !k || !v || !beta || !s || !o) return WB_EINVAL;
    if (st->d.kind != WB_BITALLOC || st->d.mode == WB_EF) return WB_EUNSUPPORTED;
    if (factor < WB_GAMMA_ERASURE || factor > WB_GAMMA_HC || C < 1) return WB_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(beta) || !aligned4(s))
        return WB_EALIGN;
    wb::AllocArgs a;
    a.state = st->state;
    a.region_stride = st->region_stride;
    a.r_default = float(1.0 / (3.0 * st->d.dk));
    a.bbar = st->d.bbar;
    a.bmin = st->d.bmin;
    a.bmax = st->d.bmax;
    a.est = st->est;
    a.factor = factor;
    a.cadence = C;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.sd = s;
    a.o = o;
    a.s_per_row = st->d.decay == WB_DECAY_PER_ROW;
    a.code_cap = int(code_capacity(st->d));
    a.t = t;
    a.seed = st->d.seed;
    if (st->d.budget == WB_BUDGET_LAYER) {
        a.H = st->d.H;
        a.rows_per_seq = st->d.H * st->d.dk;
        a.ws_c = reinterpret_cast<double*>(st->state + st->regions_bytes);
        a.ws_w = st->state + st->regions_bytes + size_t(st->d.B) * st->d.H * st->d.dk * 8;
    }
    return hip_status(wb::launch_step_allocate(st->d, a, static_cast<hipStream_t>(stream)));
}

int state_prefill_chunk(wb_state* st, const uint16_t* q_bf16, const uint16_t* k_bf16, const uint16_t* v_bf16,
                        const float* beta, const float* s, float* o, int T, int chunk, int C, uint64_t t0,
                        void* stream) {
    if (!st || !q_bf16 || !k_bf16 || !v_bf16 || !beta || !s || !o) return WB_EINVAL;
    if (T < 1 || C < 1 || chunk < 1) return WB_EINVAL;
    if (!aligned16(q_bf16) || !aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(o) || !aligned4(beta) ||
        !aligned4(s))
        return WB_EALIGN;
    wb::PrefillArgs a;
    a.base = base_args(st);
    a.q = q_bf16;
    a.k = k_bf16;
    a.v = v_bf16;
    a.beta = beta;
    a.s = s;
    a.o = o;
    a.T = T;
    a.chunk = chunk;
    a.C = C;
    a.t0 = t0;
    const hipError_t e = wb::launch_prefill(st->d, a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return WB_EUNSUPPORTED;
    return hip_status(e);
}

int state_export(const wb_state* st, void** dev_state, size_t* bytes, void** dev_side) {
    if (!st || !dev_state || !bytes || !dev_side) return WB_EINVAL;
    *dev_state = st->state;
    *bytes = st->state_bytes;
    *dev_side = st->side;
    return WB_OK;
}

int state_damp_select(const float* samples, int N, int H, int dk, int dv, int block, int k_hi, const float* s,
                      float tau, float* cost_out, uint8_t* perm_out, void* stream) {
    if (!samples || !s || !perm_out || N < 1 || H < 1) return WB_EINVAL;
    if (dk != 128 || dv != 128) return WB_EUNSUPPORTED;
    if (block != 32 && block != 64 && block != 128) return WB_EUNSUPPORTED;
    if (k_hi < 0 || k_hi > dk || !(tau > 0.f)) return WB_EINVAL;
    if (!aligned16(samples) || !aligned4(s) || (cost_out && !aligned4(cost_out))) return WB_EALIGN;
    wb::DampArgs a;
    a.samples = samples;
    a.s = s;
    a.cost = cost_out;
    a.perm = perm_out;
    a.N = N;
    a.H = H;
    a.block = block;
    a.k_hi = k_hi;
    a.tau = tau;
    return hip_status(wb::launch_damp_select(a, static_cast<hipStream_t>(stream)));
}

const char* state_status_str(int status) {
    switch (status) {
        case WB_OK: return "ok";
        case WB_EINVAL: return "invalid argument";
        case WB_ESIZE: return "buffer smaller than the layout needs";
        case WB_EUNSUPPORTED: return "unsupported shape, layout or mode";
        case WB_ELAUNCH: return "HIP launch or copy failed";
        case WB_EALIGN: return "device pointer not 16-byte aligned";
        case WB_ESCRATCH: return "layer workspace larger than the library's static scratch (16 MiB)";
        default: return "unknown status";
    }
}

}  // extern "C"
