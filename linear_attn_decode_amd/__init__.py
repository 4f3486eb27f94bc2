"""Python binding of the quantized recurrent-state write-back library.

Argument marshalling only: every step of the write-back path runs in the HIP kernels
of ``libwbstate.so`` (C ABI: ``include/wbstate.h``). PyTorch provides device memory
and streams. The binding checks tensor shapes, dtypes and devices (the C ABI takes
plain pointers and trusts sizes), then forwards pointers and the current stream.

There is no CPU fallback: if ``libwbstate.so`` is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwbstate.so")

# layout kinds, write-back rules and decay kinds (values of include/wbstate.h)
FP32, UNIFORM, HAD_INT8, MIXED, BITALLOC, HEADALLOC = 0, 1, 2, 3, 4, 5
KIND_NAMES = {"fp32": FP32, "uniform": UNIFORM, "had_int8": HAD_INT8, "mixed": MIXED, "bitalloc": BITALLOC,
              "headalloc": HEADALLOC}
RTN, SR, EF, DIR, RESQ = 0, 1, 2, 3, 4
MODE_NAMES = {"rtn": RTN, "sr": SR, "ef": EF, "dir": DIR, "resq": RESQ}
GAMMA_CODES = {"erasure": 0, "w1": 1, "hC": 2}
BUDGET_CODES = {"head": 0, "layer": 1}
DECAY_PER_HEAD, DECAY_PER_ROW = 0, 1

STATUS = {0: "ok", -1: "EINVAL", -2: "ESIZE", -3: "EUNSUPPORTED", -4: "ELAUNCH", -5: "EALIGN", -6: "ESCRATCH"}


class LayoutDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("mode", ctypes.c_int32), ("decay", ctypes.c_int32),
                ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("block", ctypes.c_int32), ("k_hi", ctypes.c_int32),
                ("bbar", ctypes.c_int32), ("bmin", ctypes.c_int32), ("bmax", ctypes.c_int32),
                ("mem_bits", ctypes.c_int32), ("budget", ctypes.c_int32), ("int_bits", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int
_U64 = ctypes.c_uint64
_F = ctypes.c_float

SIGNATURES = {
    "state_bytes": (_I, [ctypes.POINTER(LayoutDesc), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "state_alloc": (_I, [ctypes.POINTER(LayoutDesc), _P, _SZ, _P, _SZ, _P, _P, ctypes.POINTER(_P)]),
    "state_free": (_I, [_P]),
    "state_step_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _U64, _P]),
    "state_prefill_chunk": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _U64, _P]),
    "state_allocate_bits": (_I, [_P, _P, _P, _I, _I, _P]),
    "state_allocate_bits_static": (_I, [_P, _P, _P, _I, _I, _P]),
    "state_set_estimators": (_I, [_P, _P]),
    "state_step_decode_alloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _U64, _I, _I, _P]),
    "state_dequant": (_I, [_P, _P, _P]),
    "state_quantize": (_I, [_P, _P, _P]),
    "state_export": (_I, [_P, ctypes.POINTER(_P), ctypes.POINTER(_SZ), ctypes.POINTER(_P)]),
    "state_damp_select": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _F, _P, _P, _P]),
    "state_set_activity": (_I, [_P, _P, _P]),
    "state_status_str": (ctypes.c_char_p, [_I]),
}

_lib = None


def lib():
    """Load ``libwbstate.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m linear_attn_decode_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(status: int, what: str = "") -> None:
    if status != 0:
        msg = lib().state_status_str(status).decode()
        raise RuntimeError(f"{what}: {STATUS.get(status, status)} ({msg})")


def make_desc(kind, mode, B, H, dk=128, dv=128, per_row_decay=True, bits=4, block=32, k_hi=16,
              bbar=4, bmin=2, bmax=8, seed=0, mem_bits=0, budget="head", int_bits=0) -> LayoutDesc:
    kind = KIND_NAMES.get(kind, kind)
    mode = MODE_NAMES.get(mode, mode)
    return LayoutDesc(kind=kind, mode=mode, decay=DECAY_PER_ROW if per_row_decay else DECAY_PER_HEAD,
                      B=B, H=H, dk=dk, dv=dv, bits=bits, block=block, k_hi=k_hi, bbar=bbar,
                      bmin=bmin, bmax=bmax, mem_bits=mem_bits, budget=BUDGET_CODES.get(budget, budget),
                      int_bits=int_bits, seed=seed)


def buffer_sizes(desc: LayoutDesc):
    sb, side = _SZ(), _SZ()
    check(lib().state_bytes(ctypes.byref(desc), ctypes.byref(sb), ctypes.byref(side)), "state_bytes")
    return sb.value, side.value


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return _P(s.cuda_stream)


def _ptr(t, dtype, shape, name):
    import torch
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} device={t.device} contiguous={t.is_contiguous()}")
    return _P(t.data_ptr())


class WriteBackState:
    """Stored states of one layer (B x H heads) in caller-owned device memory.

    The device buffers are torch tensors owned by this object; the library writes the
    zero state into them and keeps only a host handle.
    """

    def __init__(self, kind, mode="rtn", B=1, H=1, dk=128, dv=128, per_row_decay=True, bits=4,
                 block=32, k_hi=16, bbar=4, bmin=2, bmax=8, seed=0, perm=None, device="cuda",
                 stream=None, mem_bits=0, budget="head", int_bits=0):
        import numpy as np
        import torch
        self.desc = make_desc(kind, mode, B, H, dk, dv, per_row_decay, bits, block, k_hi, bbar, bmin,
                              bmax, seed, mem_bits, budget, int_bits)
        nbytes, side = buffer_sizes(self.desc)
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.side = torch.empty(max(side // 4, 4), dtype=torch.float32, device=device)
        self.side_bytes = side
        perm_p = None
        self._perm = None
        if perm is not None:
            self._perm = np.ascontiguousarray(np.asarray(perm, dtype=np.uint8).reshape(H, dk))
            perm_p = self._perm.ctypes.data_as(_P)
        handle = _P()
        check(lib().state_alloc(ctypes.byref(self.desc), _P(self.state.data_ptr()), nbytes,
                                _P(self.side.data_ptr()) if side else None, side, perm_p,
                                _stream(stream), ctypes.byref(handle)), "state_alloc")
        self.handle = handle
        d = self.desc
        self.B, self.H, self.dk, self.dv = d.B, d.H, d.dk, d.dv

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.state_free(h)
            self.handle = None

    # -- calls -------------------------------------------------------------------
    def step_decode(self, q, k, v, beta, s, o, t: int, stream=None):
        import torch
        B, H, dk, dv = self.B, self.H, self.dk, self.dv
        s_shape = (B, H, dk) if self.desc.decay == DECAY_PER_ROW else (B, H)
        f = torch.float32
        check(lib().state_step_decode(
            self.handle, _ptr(q, f, (B, H, dk), "q"), _ptr(k, f, (B, H, dk), "k"),
            _ptr(v, f, (B, H, dv), "v"), _ptr(beta, f, (B, H), "beta"), _ptr(s, f, s_shape, "s"),
            _ptr(o, f, (B, H, dv), "o"), _U64(t), _stream(stream)), "state_step_decode")

    def step_decode_alloc(self, q, k, v, beta, s, o, t: int, factor="erasure", C=1, stream=None):
        """One decode token (index t) whose write-back allocates widths for the updated
        state (BITALLOC, RTN or SR, at the state's budget)."""
        import torch
        B, H, dk, dv = self.B, self.H, self.dk, self.dv
        s_shape = (B, H, dk) if self.desc.decay == DECAY_PER_ROW else (B, H)
        f = torch.float32
        check(lib().state_step_decode_alloc(
            self.handle, _ptr(q, f, (B, H, dk), "q"), _ptr(k, f, (B, H, dk), "k"),
            _ptr(v, f, (B, H, dv), "v"), _ptr(beta, f, (B, H), "beta"), _ptr(s, f, s_shape, "s"),
            _ptr(o, f, (B, H, dv), "o"), _U64(t), GAMMA_CODES[factor], int(C), _stream(stream)),
              "state_step_decode_alloc")

    def prefill(self, q, k, v, beta, s, o, T: int, chunk: int = 64, C: int = 8, t0: int = 0, stream=None):
        import torch
        B, H, dk, dv = self.B, self.H, self.dk, self.dv
        s_shape = (B, T, H, dk) if self.desc.decay == DECAY_PER_ROW else (B, T, H)
        bf = torch.uint16 if hasattr(torch, "uint16") else torch.int16
        check(lib().state_prefill_chunk(
            self.handle, _ptr(q.view(bf), bf, (B, T, H, dk), "q"), _ptr(k.view(bf), bf, (B, T, H, dk), "k"),
            _ptr(v.view(bf), bf, (B, T, H, dv), "v"), _ptr(beta, torch.float32, (B, T, H), "beta"),
            _ptr(s, torch.float32, s_shape, "s"), _ptr(o, torch.float32, (B, T, H, dv), "o"),
            T, chunk, C, _U64(t0), _stream(stream)), "state_prefill_chunk")

    def allocate_bits(self, s=None, r=None, factor="erasure", C=1, stream=None):
        """Allocation pass (BITALLOC). ``s``, ``r``: float32 [B, H, dk]; ``s`` None takes
        s and r from the attached estimators. ``factor``: "erasure", "w1" or "hC"."""
        import torch
        shape = (self.B, self.H, self.dk)
        check(lib().state_allocate_bits(
            self.handle, None if s is None else _ptr(s, torch.float32, shape, "s"),
            None if r is None else _ptr(r, torch.float32, shape, "r"), GAMMA_CODES[factor], int(C),
            _stream(stream)), "state_allocate_bits")

    def allocate_bits_static(self, s=None, r=None, factor="erasure", C=1, stream=None):
        """``allocate_bits`` with the workspace in the library's static device scratch
        (no allocation; calls on one GPU must not overlap)."""
        import torch
        shape = (self.B, self.H, self.dk)
        check(lib().state_allocate_bits_static(
            self.handle, None if s is None else _ptr(s, torch.float32, shape, "s"),
            None if r is None else _ptr(r, torch.float32, shape, "r"), GAMMA_CODES[factor], int(C),
            _stream(stream)), "state_allocate_bits_static")

    def set_estimators(self, est=None):
        """Attach (or with None detach) the online estimators: float32 [B, H, 2 dk + 4],
        zeroed by the caller at a sequence start; later decode steps fold their token in."""
        import torch
        p = None if est is None else _ptr(est, torch.float32, (self.B, self.H, 2 * self.dk + 4), "est")
        self._est = est
        check(lib().state_set_estimators(self.handle, p), "state_set_estimators")

    def dequant(self, S, stream=None):
        import torch
        check(lib().state_dequant(self.handle, _ptr(S, torch.float32, (self.B, self.H, self.dk, self.dv), "S"),
                                  _stream(stream)), "state_dequant")

    def quantize(self, S, stream=None):
        import torch
        check(lib().state_quantize(self.handle, _ptr(S, torch.float32, (self.B, self.H, self.dk, self.dv), "S"),
                                   _stream(stream)), "state_quantize")

    def region_stride(self) -> int:
        """Bytes between heads: the state buffer less what follows the regions (the
        MIXED permutation table; the layer-budget allocation workspace)."""
        def r256(n):
            return (n + 255) // 256 * 256
        tail = 0
        if self.desc.kind == MIXED:
            tail = r256(self.H * self.dk)
        elif self.desc.kind == BITALLOC and self.desc.budget == BUDGET_CODES["layer"]:
            tail = r256(self.B * self.H * self.dk * 9)
        elif self.desc.kind == HEADALLOC:
            tail = r256(self.B * self.H * 9)
        return (self.state.numel() - tail) // (self.B * self.H)

    def regions(self):
        """The stored bytes as a [B*H, region_stride] uint8 tensor view."""
        st = self.region_stride()
        return self.state[: st * self.B * self.H].view(self.B * self.H, st)

    def residuals(self):
        """The auxiliary write-back state [B, H, dk, dv] -- error-feedback residuals (EF),
        k-bit residual values (RESQ) or direction counters (DIR) -- or None."""
        if not self.side_bytes:
            return None
        return self.side[: self.side_bytes // 4].view(self.B, self.H, self.dk, self.dv)

    def set_activity(self, counters=None, votes=None):
        """Count write activity (UNIFORM): later decode steps add, per head, [dead-zone
        elements, level changes, votes, direction triggers, sub-threshold writes,
        same-sign vote transitions, opposite-sign vote transitions, runs started] into
        ``counters`` (int32 [B, H, 8]); ``votes`` (uint8 [B, H, dk, dv]) carries each
        element's previous vote. Both zeroed by the caller at a sequence start; both
        None stops."""
        import torch
        pc = pv = None
        if counters is not None:
            pc = _ptr(counters, torch.int32, (self.B, self.H, 8), "counters")
        if votes is not None:
            pv = _ptr(votes, torch.uint8, (self.B, self.H, self.dk, self.dv), "votes")
        self._activity = (counters, votes)
        check(lib().state_set_activity(self.handle, pc, pv), "state_set_activity")


def damp_select(samples, s, k_hi=16, block=32, tau=0.01, stream=None):
    """DAMP calibration on the GPU: samples float32 [N, H, dk, dv], s float32 [H, dk].
    Returns (perm uint8 [H, dk], cost float32 [H, dk]) as device tensors."""
    import torch
    N, H, dk, dv = samples.shape
    perm = torch.empty((H, dk), dtype=torch.uint8, device=samples.device)
    cost = torch.empty((H, dk), dtype=torch.float32, device=samples.device)
    check(lib().state_damp_select(_ptr(samples, torch.float32, (N, H, dk, dv), "samples"), N, H, dk, dv,
                                  block, k_hi, _ptr(s, torch.float32, (H, dk), "s"), _F(tau),
                                  _P(cost.data_ptr()), _P(perm.data_ptr()), _stream(stream)),
          "state_damp_select")
    return perm, cost
