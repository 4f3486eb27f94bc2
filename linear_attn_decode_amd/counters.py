"""Per-kernel means of rocprofv3 counter runs (``--pmc ...``) and the figures derived
from them, as a markdown table.

    python -m linear_attn_decode_amd.counters --kernel bitalloc_step_kernel DIR [DIR ...]

Every DIR is one rocprofv3 output directory (``-d DIR -o t --output-format csv``). For
each counter, the mean over the dispatches of the kernel whose name contains
``--kernel``. Derived figures (MI355X: 256 compute units of 4 SIMDs in 8 XCDs; a
dispatch's GRBM_GUI_ACTIVE is the sum over the 8 XCDs, so the dispatch's active cycles
are GRBM_GUI_ACTIVE / 8):
  VALU instructions per wave      SQ_INSTS_VALU / SQ_WAVES
  VALU busy                       4 SQ_ACTIVE_INST_VALU / (4 CUs) / cycles
  MFMA busy                       SQ_VALU_MFMA_BUSY_CYCLES / (4 CUs) / cycles
  LDS instructions per wave       SQ_INSTS_LDS / SQ_WAVES
  LDS bank-conflict share         SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
  wave cycles waiting on LDS      SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES
(the busy figures follow the published gfx9 definitions: SQ_ACTIVE_INST_VALU counts in
units of 4 cycles, SQ_VALU_MFMA_BUSY_CYCLES in cycles, both summed over SIMDs).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os

CUS = 256
XCDS = 8


def kernel_means(directory: str, kernel: str) -> dict[str, tuple[int, float]]:
    """counter -> (dispatches, mean value) over the dispatches of ``kernel``."""
    acc: dict[str, list[float]] = {}
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"{directory}: no counter_collection.csv")
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel in r["Kernel_Name"]:
                    acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def derived(m: dict[str, float]) -> list[tuple[str, str]]:
    out = []
    waves = m.get("SQ_WAVES")
    cyc = m["GRBM_GUI_ACTIVE"] / XCDS if "GRBM_GUI_ACTIVE" in m else None
    if cyc:
        out.append(("dispatch active cycles (GRBM_GUI_ACTIVE / 8)", f"{cyc:.0f}"))
    if waves:
        for name, key in (("VALU instructions per wave", "SQ_INSTS_VALU"), ("MFMA instructions per wave", "SQ_INSTS_MFMA"),
                          ("LDS instructions per wave", "SQ_INSTS_LDS"), ("SALU instructions per wave", "SQ_INSTS_SALU")):
            if key in m:
                out.append((name, f"{m[key] / waves:.1f}"))
    if cyc and "SQ_ACTIVE_INST_VALU" in m:
        out.append(("VALU busy", f"{100 * 4 * m['SQ_ACTIVE_INST_VALU'] / (4 * CUS) / cyc:.1f} %"))
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        out.append(("MFMA busy", f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * CUS) / cyc:.1f} %"))
    if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_ACTIVE_INST_LDS"):
        out.append(("LDS bank-conflict cycles / LDS active cycles",
                    f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_ACTIVE_INST_LDS']:.3f}"))
    if "SQ_WAIT_INST_LDS" in m and m.get("SQ_WAVE_CYCLES"):
        out.append(("wave cycles waiting on LDS", f"{100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.1f} %"))
    if "SQ_WAIT_ANY" in m and m.get("SQ_WAVE_CYCLES"):
        out.append(("wave cycles waiting (any)", f"{100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1f} %"))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", required=True)
    ap.add_argument("dirs", nargs="+")
    a = ap.parse_args(argv)
    merged: dict[str, float] = {}
    print(f"| counter | run | dispatches | mean per dispatch |\n|---|---|---:|---:|")
    for d in a.dirs:
        for k, (n, v) in sorted(kernel_means(d, a.kernel).items()):
            print(f"| {k} | {os.path.basename(d.rstrip('/'))} | {n} | {v:.6g} |")
            merged.setdefault(k, v)
    print("\n| derived | value |\n|---|---:|")
    for k, v in derived(merged):
        print(f"| {k} | {v} |")


if __name__ == "__main__":
    main()
