"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

  python profile_summary.py stats   <dir with *_kernel_stats.csv>
  python profile_summary.py traffic <FETCH_SIZE dir> <WRITE_SIZE dir> <kernel regex> [copy MiB]
  python profile_summary.py counters <pmc dir> [<pmc dir> ...]

`stats` prints the per-kernel table of a --kernel-trace --stats run.
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) of a bench run that also performed a device-to-device copy of a
known size (bench.py --calibrate-copy MiB), scales the GEMM kernel's
counters by what the same counters read for that copy, and prints HBM bytes
per launch.
`counters` tabulates the GEMM kernels of several --pmc runs of one command
(MFMA busy share, LDS instructions per MFMA, bank conflicts, L2 hit rate,
memory waits, HBM bytes per launch).
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


def _rows(d: str):
    return list(csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv")))))


def counters(dirs, copy_mib: int = 512) -> None:
    """Per GEMM kernel (median over its dispatches) from --pmc runs of the
    same command: MFMA busy share, LDS use, L2 hit rate, memory waits and, when
    FETCH_SIZE / WRITE_SIZE were collected beside a copy of copy_mib MiB, HBM
    bytes per launch.  SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of the
    1024 SIMDs and GRBM_GUI_ACTIVE the active cycles of the 8 XCDs, so
    busy share = (busy / 1024) / (active / 8)."""
    vals = {}
    durs = {}
    for d in dirs:
        for r in _rows(d):
            name = r["Kernel_Name"]
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.setdefault(name, set()).add((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    med = {k: {c: statistics.median(v) for c, v in cs.items()} for k, cs in vals.items()}
    copy = [k for k in med if "copy" in k.lower() and "FETCH_SIZE" in med[k]]
    sf = sw = None
    if copy:
        cf = max(max(vals[k]["FETCH_SIZE"]) for k in copy)
        cws = [max(vals[k]["WRITE_SIZE"]) for k in copy if "WRITE_SIZE" in vals[k]]
        if cws:
            sf, sw = copy_mib * 1024.0 / cf, copy_mib * 1024.0 / max(cws)
            print("copy of %d MiB: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB -> scale %.4f / %.4f\n" % (
                copy_mib, cf, max(cws), sf, sw))
    print("| kernel | dispatches | median us | MFMA busy | LDS instr / MFMA instr | LDS bank-conflict cycles / LDS active "
          "| L2 hit | wave cycles waiting on memory | TA command FIFO full cycles | HBM read + write per launch |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for k, c in sorted(med.items(), key=lambda kv: -statistics.median([t for _, t in durs[kv[0]]])):
        if not re.search(r"gemm|skinny|preshuffle|split_reduce", k):
            continue
        us = statistics.median([t for _, t in durs[k]]) / 1e3
        f = lambda a: c.get(a)
        busy = "%.1f%%" % (100.0 * f("SQ_VALU_MFMA_BUSY_CYCLES") / 1024 / (f("GRBM_GUI_ACTIVE") / 8)) \
            if f("SQ_VALU_MFMA_BUSY_CYCLES") and f("GRBM_GUI_ACTIVE") else "-"
        ldsr = "%.3f" % (f("SQ_INSTS_LDS") / f("SQ_INSTS_MFMA")) if f("SQ_INSTS_LDS") is not None and f("SQ_INSTS_MFMA") else "-"
        bank = "%.3f" % (f("SQ_LDS_BANK_CONFLICT") / f("SQ_LDS_IDX_ACTIVE")) \
            if f("SQ_LDS_BANK_CONFLICT") is not None and f("SQ_LDS_IDX_ACTIVE") else "-"
        hit = "%.1f%%" % (100.0 * f("TCC_HIT_sum") / (f("TCC_HIT_sum") + f("TCC_MISS_sum"))) \
            if f("TCC_HIT_sum") is not None and f("TCC_MISS_sum") else "-"
        wait = "%.1f%%" % (100.0 * f("SQ_WAIT_ANY") / f("SQ_WAVE_CYCLES")) if f("SQ_WAIT_ANY") and f("SQ_WAVE_CYCLES") else "-"
        fifo = "%.3g" % f("SQ_VMEM_TA_CMD_FIFO_FULL") if f("SQ_VMEM_TA_CMD_FIFO_FULL") is not None else "-"
        hbm = "%.4g + %.4g B" % (f("FETCH_SIZE") * 1024 * sf, f("WRITE_SIZE") * 1024 * sw) \
            if sf and f("FETCH_SIZE") is not None and f("WRITE_SIZE") is not None else "-"
        print("| %s | %d | %.1f | %s | %s | %s | %s | %s | %s | %s |" % (
            k.replace("|", "/")[:100], len(durs[k]), us, busy, ldsr, bank, hit, wait, fifo, hbm))


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "counters":
        counters(sys.argv[2:])
    elif len(sys.argv) >= 5 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]) if len(sys.argv) > 5 else 512)
    else:
        print(__doc__)
        sys.exit(2)
