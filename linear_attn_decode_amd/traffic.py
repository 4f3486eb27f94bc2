"""HBM traffic of the decode kernel from rocprofv3 memory counters.

Two counter runs of ``bench.py --profile-steps N`` (one with ``--pmc FETCH_SIZE``, one
with ``--pmc WRITE_SIZE``; each counter run is its own process because the counter
blocks cannot hold both at once) are reduced here to bytes per launch of the decode
kernel. Each counter is scaled by the ratio it shows on a calibration kernel of known
traffic that the same run launches first (an elementwise negation reading and writing
``calib_bytes`` each), so the reported bytes are in the units of the algorithmic count.

    python -m linear_attn_decode_amd.traffic --fetch DIR --write DIR \\
        --workload kda-bitalloc --kernel bitalloc_step_kernel --calib-bytes N --out FILE.json

The result carries the hash of the kernel sources it was measured on; ``bench.py``
reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    """Hash of every kernel source file (csrc/), the identity of a measured kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def per_dispatch(directory: str, counter: str) -> list[tuple[str, float]]:
    """(kernel name, counter value) of every dispatch in a rocprofv3 csv directory, in
    dispatch order."""
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(name, value) for _, name, value in rows]


def scaled_bytes(directory: str, counter: str, kernel: str, calib_kernel: str, calib_bytes: float) -> dict:
    rows = per_dispatch(directory, counter)
    cal = [v for n, v in rows if calib_kernel in n]
    dec = [v for n, v in rows if kernel in n]
    if not cal or not dec:
        raise SystemExit(f"{directory}: no {counter} rows for the calibration ({len(cal)}) or the kernel ({len(dec)})")
    cal_kib = sum(cal) / len(cal)
    factor = calib_bytes / (cal_kib * 1024.0)
    mean_kib = sum(dec) / len(dec)
    return {"counter": counter, "dispatches": len(dec), "mean_kib": mean_kib, "calib_kib": cal_kib,
            "scale": factor, "bytes": mean_kib * 1024.0 * factor}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--calib-kernel", default="neg")
    ap.add_argument("--calib-bytes", type=float, required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    fetch = scaled_bytes(a.fetch, "FETCH_SIZE", a.kernel, a.calib_kernel, a.calib_bytes)
    write = scaled_bytes(a.write, "WRITE_SIZE", a.kernel, a.calib_kernel, a.calib_bytes)
    out = {"workload": a.workload, "kernel": a.kernel, "kernel_hash": kernel_source_hash(),
           "fetch": fetch, "write": write, "bytes_per_launch": fetch["bytes"] + write["bytes"],
           "calibration": {"kernel": a.calib_kernel, "bytes_read": a.calib_bytes, "bytes_written": a.calib_bytes}}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
