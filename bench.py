#!/usr/bin/env python3
"""Throughput of the fused quantized write-back decode step on one MI355X.

A step is one decode token through one layer: every head state of a B x H layer is
dequantized, advanced by the gated delta rule, read out and requantized in place
(one kernel launch), and the layer's decay-aware allocation pass runs on its cadence
(every 64 of that layer's tokens). L independent layer states are cycled so that the
working set is several times the 256 MB last-level cache; q, k, v, beta, s and o
cycle through a 64-token ring on the device. Inputs are synthetic (seeded), with the
distributions of the decode studies, and resident in HBM before timing starts.

Prints ONE JSON line: tokens/s (value), the achieved HBM bandwidth of the decode
kernel against the 8 TB/s peak (roofline), and the CPU oracle timed on a bounded sample
of the same work (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "kda-bitalloc": dict(cfg=3, kind="bitalloc", B=256, H=32, per_row=True, layers=15, alloc_every=64,
                         extra=dict(bbar=4, bmin=2, bmax=8), kernel="bitalloc_step_kernel"),
    # the same, with the span-64 decay / erasure estimators folded in by every decode
    # step and the allocation passes taking s and r from them
    "kda-bitalloc-online": dict(cfg=3, kind="bitalloc", B=256, H=32, per_row=True, layers=15, alloc_every=64,
                                extra=dict(bbar=4, bmin=2, bmax=8), kernel="bitalloc_step_kernel", online=True),
    # the same decode step under Philox stochastic rounding (the second rule of the
    # decay-aware configuration)
    "kda-bitalloc-sr": dict(cfg=3, kind="bitalloc", mode="sr", B=256, H=32, per_row=True, layers=15, alloc_every=64,
                            extra=dict(bbar=4, bmin=2, bmax=8), kernel="bitalloc_step_kernel"),
    # ... and under error feedback (a float32 residual per element read and written)
    "kda-bitalloc-ef": dict(cfg=3, kind="bitalloc", mode="ef", B=256, H=32, per_row=True, layers=15, alloc_every=64,
                            extra=dict(bbar=4, bmin=2, bmax=8), kernel="bitalloc_step_kernel"),
    "kda-mixed": dict(cfg=2, kind="mixed", B=256, H=32, per_row=True, layers=7, alloc_every=0,
                      extra=dict(block=32, k_hi=16), kernel="rot_step_kernel"),
    "gdn-had-int8": dict(cfg=1, kind="had_int8", B=64, H=16, per_row=False, layers=60, alloc_every=0,
                         extra=dict(block=128), kernel="rot_step_kernel"),
    "kda-fp32": dict(cfg=None, kind="fp32", B=256, H=32, per_row=True, layers=3, alloc_every=0, extra={},
                     kernel="wb_kernel"),
    "kda-prefill": dict(cfg=4, kind="mixed", B=8, H=32, per_row=True, layers=1, alloc_every=0, T=8192, C=8,
                        extra=dict(block=32, k_hi=16)),
    # the widened rows, timed the same way: temporal-memory write-back, write-activity
    # counters, allocation at every write-back, the layer budget, one-bit rows, the
    # per-head unit and the INT4 tier (the layer budget and one-bit rows run in the tuned
    # BITALLOC kernel, the per-head unit in its own tuned kernel, the INT4 tier in the
    # rotated-domain kernel, the rest in the generic decode kernel)
    "kda-uniform4-dir": dict(cfg=None, kind="uniform", mode="dir", B=256, H=32, per_row=True, layers=3,
                             alloc_every=0, extra=dict(bits=4, mem_bits=2), kernel="wb_kernel"),
    "kda-uniform4-activity": dict(cfg=None, kind="uniform", B=256, H=32, per_row=True, layers=3, alloc_every=0,
                                  extra=dict(bits=4), kernel="wb_kernel", activity=True),
    "kda-bitalloc-alloc-each": dict(cfg=3, kind="bitalloc", B=256, H=32, per_row=True, layers=15, alloc_every=0,
                                    extra=dict(bbar=4, bmin=2, bmax=8), kernel="allocate_kernel", online=True,
                                    alloc_each=True),
    # allocation at every write-back under the layer budget, rounding stochastically:
    # three launches per step (costs, widths per sequence, rounding at those widths)
    "kda-bitalloc-layer-sr-alloc-each": dict(cfg=3, kind="bitalloc", mode="sr", B=256, H=32, per_row=True, layers=8,
                                             alloc_every=0, extra=dict(bbar=4, bmin=2, bmax=8, budget="layer"),
                                             kernel="allocate_kernel", online=True, alloc_each=True),
    "kda-bitalloc-layer": dict(cfg=3, kind="bitalloc", B=256, H=32, per_row=True, layers=8, alloc_every=64,
                               extra=dict(bbar=4, bmin=2, bmax=8, budget="layer"), kernel="bitalloc_step_kernel"),
    "kda-bitalloc-1bit": dict(cfg=3, kind="bitalloc", B=256, H=32, per_row=True, layers=15, alloc_every=64,
                              extra=dict(bbar=4, bmin=1, bmax=8), kernel="bitalloc_step_kernel"),
    "gdn-headalloc": dict(cfg=1, kind="headalloc", B=64, H=16, per_row=False, layers=60, alloc_every=64,
                          extra=dict(bbar=4, bmin=2, bmax=8), kernel="headalloc_step_kernel"),
    "gdn-headalloc-ef": dict(cfg=1, kind="headalloc", mode="ef", B=64, H=16, per_row=False, layers=60, alloc_every=64,
                             extra=dict(bbar=4, bmin=2, bmax=8), kernel="headalloc_step_kernel"),
    "gdn-had-int4": dict(cfg=1, kind="had_int8", B=64, H=16, per_row=False, layers=60, alloc_every=0,
                         extra=dict(block=128, int_bits=4), kernel="rot_step_kernel"),
    # the rotated layouts under Philox stochastic rounding (the tuned rotated-domain kernel) ...
    "kda-mixed-sr": dict(cfg=2, kind="mixed", mode="sr", B=256, H=32, per_row=True, layers=7, alloc_every=0,
                         extra=dict(block=32, k_hi=16), kernel="rot_step_kernel"),
    "gdn-had-int8-sr": dict(cfg=1, kind="had_int8", mode="sr", B=64, H=16, per_row=False, layers=60,
                            alloc_every=0, extra=dict(block=128), kernel="rot_step_kernel"),
    # ... and under error feedback (a float32 residual per INT8 element read and written)
    "kda-mixed-ef": dict(cfg=2, kind="mixed", mode="ef", B=256, H=32, per_row=True, layers=7, alloc_every=0,
                         extra=dict(block=32, k_hi=16), kernel="rot_step_kernel"),
    "gdn-had-int8-ef": dict(cfg=1, kind="had_int8", mode="ef", B=64, H=16, per_row=False, layers=60,
                            alloc_every=0, extra=dict(block=128), kernel="rot_step_kernel"),
}
PEAK_FP64_MFMA_TFLOPS = 78.6     # the prefill's state path runs on float64 matrix cores


def prefill_flops_per_segment(L=8):
    """Float operations of one L-token segment of one head, as the prefill kernel
    evaluates it: [k^; q^] S_0 (2L x 128 x 128), the two Gram matrices (L x L x 128),
    the forward solve and outputs, the rank-L update and its decay scaling, and the
    three 128-point transforms per output vector of the rotated rows."""
    d = 128
    contraction = 2 * (2 * L) * d * d
    update = 2 * d * d * L + d * d
    gram = 2 * 2 * L * L * d
    solve = 2 * d * (L * (L - 1) // 2 + L * (L + 1) // 2) + 2 * d * L
    transforms = (2 * L + L) * d * 7
    mfma = contraction + update - d * d
    return contraction + update + gram + solve + transforms, mfma
DEFAULT = "kda-bitalloc"
DK = DV = 128


def region_bytes(kind, extra):
    """(read, written) bytes of one head's stored state in one decode step."""
    dk, dv = DK, DV
    ib = extra.get("int_bits") or 8
    if kind == "fp32":
        return 4 * dk * dv, 4 * dk * dv
    if kind == "uniform":
        n = dk * dv * extra["bits"] // 8
        return n, n
    if kind == "had_int8":
        n = dk * dv * ib // 8 + dk * (dv // extra["block"]) * 4
        return n, n
    if kind == "mixed":
        qr = dk - extra["k_hi"]
        n = extra["k_hi"] * dv * 2 + qr * dv * ib // 8 + qr * (dv // extra["block"]) * 4
        return n, n
    code = dk * dv * extra["bbar"] // 8              # the mean width's codes
    if kind == "headalloc":
        groups = (dk // 32) * dv
        return code + 3 * groups + 16, code + 2 * groups     # read: + scales, fits, width; write: + scales
    return code + 3 * dk, code + 2 * dk          # read: codes + Delta + meta; write: codes + Delta


def algorithmic_bytes_per_head(kind, extra, per_row, online=False, mode="rtn", activity=False):
    rd, wr = region_bytes(kind, extra)
    io = 2 * DK * 4 + DV * 4 + 4 + (DK * 4 if per_row else 4) + DV * 4
    est = 2 * (2 * DK * 4 + 4) if online else 0      # estimators read and written
    # float32 side value per element, read and written (not for the float16 rows of MIXED)
    side_rows = DK - extra.get("k_hi", 0) if kind == "mixed" else DK
    side = 2 * 4 * side_rows * DV if mode in ("ef", "dir", "resq") else 0
    votes = 2 * DK * DV + 8 * 4 if activity else 0   # vote state read and written, the counters
    return rd + wr + io + est + side + votes


def load_traffic(workload):
    path = os.path.join(ROOT, "profiles", f"{WORKLOADS[workload]['kernel']}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from linear_attn_decode_amd.traffic import kernel_source_hash
    if t.get("kernel_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def warm_states(wb, torch, w, seed):
    """L layer states holding a realistic state: rows of widely different ranges,
    slow-decay rows larger; BITALLOC states get one allocation pass."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 100)
    B, H = w["B"], w["H"]
    perm = None
    if w["kind"] == "mixed":
        import numpy as np
        rng = np.random.default_rng(seed)
        perm = np.stack([rng.permutation(DK) for _ in range(H)])
    states = []
    for layer in range(w["layers"]):
        st = wb.WriteBackState(w["kind"], w.get("mode", "rtn"), B, H, DK, DV, w["per_row"], seed=seed + layer,
                               perm=perm, **w["extra"])
        scale = torch.exp(torch.rand((B, H, DK, 1), generator=g, device="cuda") * 3.5 - 3.0)
        S = torch.randn((B, H, DK, DV), generator=g, device="cuda") * scale
        st.quantize(S.contiguous())
        states.append(st)
        del S
    return states


def run_gpu(args, w):
    import torch

    import linear_attn_decode_amd as wb
    from synth import device_inputs

    torch.cuda.set_device(0)
    B, H = w["B"], w["H"]
    R = 64
    inp = device_inputs(args.seed, B, H, DK, DV, R, w["per_row"])
    s_ring = inp["s"].unsqueeze(0).expand((R,) + tuple(inp["s"].shape)).contiguous()
    # the allocation takes a decay per row (a per-head decay repeated over the rows)
    s_alloc = inp["s"] if w["per_row"] else inp["s"].unsqueeze(-1).expand(B, H, DK).contiguous()
    o_ring = torch.zeros((R, B, H, DV), dtype=torch.float32, device="cuda")
    states = warm_states(wb, torch, w, args.seed)
    if w["kind"] in ("bitalloc", "headalloc"):
        for st in states:
            st.allocate_bits(s_alloc)
    if w.get("activity"):
        for st in states:
            st.set_activity(torch.zeros((B, H, 8), dtype=torch.int32, device="cuda"),
                            torch.zeros((B, H, DK, DV), dtype=torch.uint8, device="cuda"))
    ests = []
    if w.get("online"):
        for st in states:
            ests.append(torch.zeros((B, H, 2 * DK + 4), dtype=torch.float32, device="cuda"))
            st.set_estimators(ests[-1])
        s_alloc = None                                # allocation from the estimators
    torch.cuda.synchronize()
    alloc_every = w["alloc_every"]
    # each layer's token counter starts at its own phase of the allocation cadence, so
    # that over the run the passes fall at the steady rate of one per `alloc_every` steps
    counts = [(layer * alloc_every) // len(states) if alloc_every else 0 for layer in range(len(states))]

    def one(i, ev_alloc=None):
        layer = i % len(states)
        r = i % R
        st = states[layer]
        if w.get("alloc_each"):
            st.step_decode_alloc(inp["q"][r], inp["k"][r], inp["v"][r], inp["beta"][r], s_ring[r], o_ring[r],
                                 counts[layer])
        else:
            st.step_decode(inp["q"][r], inp["k"][r], inp["v"][r], inp["beta"][r], s_ring[r], o_ring[r],
                           counts[layer])
        counts[layer] += 1
        if alloc_every and counts[layer] % alloc_every == 0:
            if ev_alloc is not None:
                ev_alloc[0].record()
            st.allocate_bits(s_alloc)
            if ev_alloc is not None:
                ev_alloc[1].record()
            return True
        return False

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    # Decode launches are timed in groups of G back-to-back launches (HIP events on the
    # stream the kernels run on); groups that contain an allocation pass are left out
    # of the per-launch figure, and the allocation passes are timed on their own.
    G = 16
    ev = lambda: torch.cuda.Event(enable_timing=True)
    groups = []
    alloc_evs = []
    start, end = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    g0, n, dirty = None, 0, False
    for i in range(args.steps):
        if i % G == 0:
            g0, n, dirty = ev(), 0, False
            g0.record()
        ae = (ev(), ev())
        if one(args.warmup + i, ae):
            alloc_evs.append(ae)
            dirty = True
        n += 1
        if i % G == G - 1 or i == args.steps - 1:
            g1 = ev()
            g1.record()
            groups.append((g0, g1, n, dirty))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    clean = [(a.elapsed_time(b), n) for a, b, n, d in groups if not d]
    dec_ms = [t / n for t, n in clean for _ in range(n)]
    alloc_ms = [a.elapsed_time(b) for a, b in alloc_evs]
    in_window = len(alloc_ms)
    if alloc_every and in_window < 3:
        # a short run holds fewer passes than it should at the cadence: time a few more
        # (after the window) for the per-pass cost that is amortised into the result
        for i in range(3 - in_window):
            ae = (ev(), ev())
            ae[0].record()
            states[i % len(states)].allocate_bits(s_alloc)
            ae[1].record()
            alloc_evs.append(ae)
        torch.cuda.synchronize()
        alloc_ms = [a.elapsed_time(b) for a, b in alloc_evs]
    return {"total_ms": total_ms, "wall_s": wall, "decode_ms": dec_ms, "alloc_ms": alloc_ms,
            "alloc_in_window": in_window, "states": states, "inputs": inp}


def run_prefill(args, w):
    import numpy as np
    import torch

    import linear_attn_decode_amd as wb
    from synth import device_inputs

    torch.cuda.set_device(0)
    B, H, T, C = w["B"], w["H"], w["T"], w["C"]
    rng = np.random.default_rng(args.seed)
    perm = np.stack([rng.permutation(DK) for _ in range(H)])
    st = wb.WriteBackState(w["kind"], "rtn", B, H, DK, DV, w["per_row"], perm=perm, **w["extra"])
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed + 7)

    def bf16(x):
        return x.to(torch.bfloat16).view(torch.int16)

    def unit(shape):
        x = torch.randn(shape, generator=g, device="cuda")
        return x / x.norm(dim=-1, keepdim=True)

    q = bf16(unit((B, T, H, DK)))
    k = bf16(unit((B, T, H, DK)))
    v = bf16(torch.randn((B, T, H, DV), generator=g, device="cuda"))
    beta = torch.rand((B, T, H), generator=g, device="cuda")
    s_h = device_inputs(args.seed, 1, H, DK, DV, 1, True)["s"][0]
    s = s_h.view(1, 1, H, DK).expand(B, T, H, DK).contiguous()
    o = torch.zeros((B, T, H, DV), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(args.warmup):
        st.prefill(q, k, v, beta, s, o, T, 64, C, 0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        st.prefill(q, k, v, beta, s, o, T, 64, C, 0)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in evs]
    return {"ms": ms, "wall_s": wall, "state": st, "perm": perm}


def cpu_baseline(w, gpu, budget_s):
    """The oracle, single-threaded, on a bounded sample of the same decode work: the
    stored regions of sampled heads after the GPU warm-up, one step each."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    from oracle import layouts as L
    from oracle.estimators import ema_fold, ema_init
    from oracle.step import decode_step

    st = gpu["states"][0]
    inp = gpu["inputs"]
    lay = L.Layout(kind=w["kind"], B=w["B"], H=w["H"], dk=DK, dv=DV, per_row_decay=w["per_row"], mode="rtn",
                   **{k: v for k, v in w["extra"].items()})
    regs = st.regions()
    perm = st._perm
    q = inp["q"][0].cpu().numpy()
    k = inp["k"][0].cpu().numpy()
    v = inp["v"][0].cpu().numpy()
    beta = inp["beta"][0].cpu().numpy()
    s = inp["s"].cpu().numpy()
    rng = np.random.default_rng(0)
    order = rng.permutation(w["B"] * w["H"])
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    n = 0
    t0 = time.perf_counter()
    try:
        if ctx:
            ctx.__enter__()
        while True:
            idx = int(order[n % order.size])
            b, h = divmod(idx, w["H"])
            reg = regs[idx].cpu().numpy()[: lay.region_size()]
            decode_step(lay, reg, None, q[b, h], k[b, h], v[b, h], beta[b, h], s[b, h], 0, b, h,
                        None if perm is None else perm[h])
            if w.get("online"):
                ema_fold(ema_init(DK), s[b, h], float(beta[b, h]), k[b, h])
            n += 1
            if time.perf_counter() - t0 >= budget_s and n >= 4:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    el = time.perf_counter() - t0
    per_head = el / n
    tok_s = 1.0 / (per_head * w["H"])          # one token of a sequence = H heads
    return {"value": tok_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {w['B'] * w['H']} head states of one decode step, float64 numpy, "
                      f"{el:.1f} s, extrapolated to the full step (host has {os.cpu_count()} logical CPUs)"}


CALIB_BYTES = 256 * 1024 * 1024


def profile_run(args, w):
    """For the memory-counter runs: one elementwise negation of a 256 MiB buffer (reads
    and writes CALIB_BYTES each; the traffic reducer scales the counters by it), then
    `profile_steps` decode steps of the workload, cycling the layer states as the
    timed run does."""
    import torch

    args.steps, args.warmup = args.profile_steps, 0
    x = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y
    run_gpu(args, w)
    torch.cuda.synchronize()
    print(json.dumps({"profile_steps": args.profile_steps, "workload": args.workload, "kernel": w["kernel"],
                      "calib_bytes": CALIB_BYTES}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="counter run: a calibration kernel of known traffic, then this many decode steps "
                         "(no timing, no JSON result line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the write-back runs on one GPU's "
              f"share of the heads (every head state is independent, so several GPUs would each take a "
              f"disjoint set of (sequence, head) pairs with no communication).", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    if args.profile_steps:
        return profile_run(args, w)
    if args.workload == "kda-prefill":
        return main_prefill(args, w)
    gpu = run_gpu(args, w)
    B, H = w["B"], w["H"]
    K = args.steps
    total_s = gpu["total_ms"] / 1e3
    tokens = B * K
    dec = sorted(gpu["decode_ms"])
    avg_dec_ms = sum(dec) / len(dec)
    bytes_launch = algorithmic_bytes_per_head(w["kind"], w["extra"], w["per_row"], w.get("online", False),
                                              w.get("mode", "rtn"), w.get("activity", False)) * B * H
    achieved = bytes_launch / (avg_dec_ms / 1e3) / 1e9
    traffic = load_traffic(args.workload)
    # Whole-job time: the timed window, with the allocation passes counted at their
    # cadence (one per `alloc_every` layer tokens): the passes inside the window are in
    # it; the difference to the steady-rate count K / alloc_every is added (or taken
    # away) at the measured per-pass time.
    alloc_ms = gpu["alloc_ms"]
    pass_ms = sum(alloc_ms) / len(alloc_ms) if alloc_ms else 0.0
    n_in = gpu["alloc_in_window"]
    expected = K / w["alloc_every"] if w["alloc_every"] else 0.0
    job_s = total_s + (expected - n_in) * pass_ms / 1e3
    out = {
        "metric": "write-back decode tokens/s + effective HBM GB/s (% peak), 32h x 128x128, B=256",
        "value": tokens / job_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": job_s * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if w["kind"] in ("had_int8", "mixed") else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: decode write-back, {w['kind']} layout, B={B}, H={H}, "
                               f"dk=dv=128, {'per-row' if w['per_row'] else 'per-head'} decay, "
                               f"{w.get('mode', 'rtn').upper()}, "
                               f"{w['layers']} layer states cycled"
                               + (f", allocation pass every {w['alloc_every']} tokens per layer" if w["alloc_every"] else "")
                               + (", span-64 decay/erasure estimators folded in every step, allocation from them"
                                  if w.get("online") else ""),
                   "global_batch": B, "heads": H, "layers_cycled": w["layers"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": w["kernel"], "bytes_per_launch": bytes_launch,
                     "avg_launch_us": avg_dec_ms * 1e3, "median_launch_us": dec[len(dec) // 2] * 1e3,
                     "timing": "HIP events around groups of 16 back-to-back decode launches"},
        "allocation_pass": {"every_tokens_per_layer": w["alloc_every"] or None,
                            "launches_in_window": n_in, "launches_at_cadence": expected,
                            "avg_us": pass_ms * 1e3 if alloc_ms else None,
                            "amortised_us_per_step": (pass_ms * 1e3 / w["alloc_every"]) if w["alloc_every"] else 0.0,
                            "window_tokens_per_s": tokens / total_s},
        "wall_s": gpu["wall_s"],
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, gpu, args.cpu_budget)
    print(json.dumps(out), flush=True)


def main_prefill(args, w):
    gpu = run_prefill(args, w)
    B, H, T, C = w["B"], w["H"], w["T"], w["C"]
    ms = sorted(gpu["ms"])
    avg = sum(ms) / len(ms)
    seg = T // 8
    flops, mfma_flops = prefill_flops_per_segment(8)
    total = flops * seg * B * H
    achieved = total / (avg / 1e3) / 1e12
    out = {
        "metric": "chunked prefill with deferred write-back tokens/s",
        "value": B * T / (avg / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": avg,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"kda-prefill: B={B}, H={H}, T={T}, dk=dv=128, per-row decay, mixed layout "
                               f"(16 float16 rows + Hadamard INT8, 32-value blocks), write-back every {C} tokens",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP64_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP64_MFMA_TFLOPS, "traffic": None, "kernel": "prefill_kernel",
                     "flops_per_launch": total, "mfma_flops_per_launch": mfma_flops * seg * B * H,
                     "avg_launch_us": avg * 1e3},
        "wall_s": gpu["wall_s"],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
