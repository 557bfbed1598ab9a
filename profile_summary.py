"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

  python profile_summary.py stats   <dir with *_kernel_stats.csv>
  python profile_summary.py traffic <FETCH_SIZE dir> <WRITE_SIZE dir> <kernel regex> [copy MiB]

`stats` prints the per-kernel table of a --kernel-trace --stats run.
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) of a bench run that also performed a device-to-device copy of a
known size (bench.py --calibrate-copy MiB), scales the GEMM kernel's
counters by what the same counters read for that copy, and prints HBM bytes
per launch.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources that define the timed GEMM kernel; a traffic figure is valid only
# for the exact sources it was measured on.
KERNEL_SOURCES = ["tiled_gemm_amd/csrc/gemm_pipe.hip", "tiled_gemm_amd/csrc/device.hpp",
                  "tiled_gemm_amd/csrc/layout.hpp", "tiled_gemm_amd/csrc/kernels.hpp"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(path: str):
    """TRAFFIC_BYTES from a committed summary, or None if the kernel sources
    changed since it was measured."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] in ("TRAFFIC_BYTES", "SOURCE_SHA"):
            vals[parts[0]] = parts[1]
    if vals.get("SOURCE_SHA") != kernel_source_sha() or "TRAFFIC_BYTES" not in vals:
        return None
    return float(vals["TRAFFIC_BYTES"])


def _one(pattern: str) -> str:
    files = glob.glob(pattern)
    if not files:
        raise SystemExit("no file matches %s" % pattern)
    return files[0]


def stats(d: str) -> None:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*kernel_stats.csv")))))
    print("| kernel | calls | avg us | min us | max us | % time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            r["Name"].replace("|", "/"), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


def _counter(d: str, name: str):
    out = []
    for r in csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv")))):
        if r["Counter_Name"] == name:
            out.append((r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])))
    return out


def traffic(fetch_dir: str, write_dir: str, kernel_re: str, copy_mib: int = 512) -> None:
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0

    def copy_vals(rows):
        # the calibration copy: the largest copy-kernel dispatch
        vals = [v for n, v, g in rows if "copy" in n.lower()]
        return max(vals) if vals else None

    cf, cw = copy_vals(fetch), copy_vals(write)
    rx = re.compile(kernel_re)
    gf = [v for n, v, g in fetch if rx.search(n)]
    gw = [v for n, v, g in write if rx.search(n)]
    if not gf or not gw or cf is None or cw is None:
        raise SystemExit("missing kernel or copy dispatches")
    sf, sw = copy_kib / cf, copy_kib / cw
    mf, mw = statistics.median(gf), statistics.median(gw)
    print("copy of %d MiB: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB -> scale %.4f / %.4f" % (
        copy_mib, cf, cw, sf, sw))
    print("kernel /%s/: %d dispatches, median FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB" % (
        kernel_re, len(gf), mf, mw))
    hbm = (mf * sf + mw * sw) * 1024.0
    print("HBM bytes per launch (scaled): read %.0f + write %.0f = %.0f" % (
        mf * sf * 1024, mw * sw * 1024, hbm))
    print("TRAFFIC_BYTES %.0f" % hbm)
    print("SOURCE_SHA %s" % kernel_source_sha())


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) >= 5 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]) if len(sys.argv) > 5 else 512)
    else:
        print(__doc__)
        sys.exit(2)
