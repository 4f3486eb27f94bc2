"""Seeded synthetic inputs for the gated delta-rule write-back step.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It draws random numbers and nothing else: it holds none of the method's
arithmetic (no recurrence, quantizer, transform or allocation).

Distributions (the workloads of the decode and prefill studies):
  * keys and queries: a standard-normal vector per (t, b, h), divided by its L2
    norm (computed in float64, then cast to float32);
  * values: standard normal;
  * beta: uniform on [0, 1) per (t, b, h);
  * decay rate s: log-uniform on [1e-3, 1], drawn once per (head, key row) for
    per-row decay (KDA) or once per head for per-head decay (GDN); it is held
    constant over time and shared by every sequence of the batch.

Two generators are offered: ``decode_inputs`` (numpy PCG64, bit-reproducible on any
host, used wherever the oracle must see the same values) and ``device_inputs``
(torch on a GPU, for full-size timing runs; parity subsets copy it to the host).
"""
from __future__ import annotations

import numpy as np

S_MIN = 1e-3
S_MAX = 1.0


def _unit_rows(g: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(g * g, axis=-1, keepdims=True))
    return (g / n).astype(np.float32)


def decay_rates(rng: np.random.Generator, H: int, dk: int, per_row: bool) -> np.ndarray:
    """Log-uniform decay rates: [H, dk] when per_row else [H]."""
    shape = (H, dk) if per_row else (H,)
    u = rng.random(shape)
    return np.exp(np.log(S_MIN) + u * (np.log(S_MAX) - np.log(S_MIN))).astype(np.float32)


def decode_inputs(seed: int, B: int, H: int, dk: int, dv: int, T: int,
                  per_row_decay: bool = True) -> dict:
    """Inputs for T decode tokens.

    Returns float32 arrays q, k [T, B, H, dk]; v [T, B, H, dv]; beta [T, B, H];
    s [B, H, dk] (per-row) or [B, H] (per-head), constant over t.
    """
    rng = np.random.default_rng(seed)
    s_h = decay_rates(rng, H, dk, per_row_decay)
    k = _unit_rows(rng.standard_normal((T, B, H, dk)))
    q = _unit_rows(rng.standard_normal((T, B, H, dk)))
    v = rng.standard_normal((T, B, H, dv)).astype(np.float32)
    beta = rng.random((T, B, H)).astype(np.float32)
    s = np.broadcast_to(s_h, (B,) + s_h.shape).copy()
    return {"q": q, "k": k, "v": v, "beta": beta, "s": s}


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def prefill_inputs(seed: int, B: int, H: int, dk: int, dv: int, T: int,
                   per_row_decay: bool = True) -> dict:
    """Inputs for one prefill call of T tokens, token-major as the kernel takes them.

    q, k, v are bfloat16 bit patterns (uint16) [B, T, H, d]; beta float32 [B, T, H];
    s float32 [B, T, H, dk] (per-row) or [B, T, H]; the decay rates are constant
    over t and shared over the batch.
    """
    rng = np.random.default_rng(seed)
    s_h = decay_rates(rng, H, dk, per_row_decay)
    k = _unit_rows(rng.standard_normal((B, T, H, dk)))
    q = _unit_rows(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    s = np.broadcast_to(s_h, (B, T) + s_h.shape).copy()
    return {"q": to_bf16(q), "k": to_bf16(k), "v": to_bf16(v), "beta": beta, "s": s}


def device_inputs(seed: int, B: int, H: int, dk: int, dv: int, T: int,
                  per_row_decay: bool = True, device: str = "cuda"):
    """Same distributions as ``decode_inputs``, drawn on the GPU with torch.

    Used for full-size timing rings; the values differ from ``decode_inputs`` (a
    different generator), so parity tests copy these tensors to the host.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    u = torch.rand((H, dk) if per_row_decay else (H,), generator=g, device=device,
                   dtype=torch.float64)
    s_h = torch.exp(np.log(S_MIN) + u * (np.log(S_MAX) - np.log(S_MIN))).to(f32)

    def unit(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
        return (x / x.norm(dim=-1, keepdim=True)).to(f32)

    k = unit((T, B, H, dk))
    q = unit((T, B, H, dk))
    v = torch.randn((T, B, H, dv), generator=g, device=device, dtype=f32)
    beta = torch.rand((T, B, H), generator=g, device=device, dtype=f32)
    s = s_h.unsqueeze(0).expand((B,) + tuple(s_h.shape)).contiguous()
    return {"q": q, "k": k, "v": v, "beta": beta, "s": s}
