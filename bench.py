"""Benchmark of the tiled GEMM on one MI355X.

A step is one gemm_run of C = A * B^T on the headline workload: bf16
8192 x 8192 x 8192 with B pre-shuffled into MFMA operand order (the
pre-shuffle is done once, ahead of the timed steps, and reported separately),
fp32 accumulation, bf16 output.  Inputs are seeded synthetic data resident in
HBM before timing starts.

Prints one JSON line with TFLOP/s, the roofline of the GEMM kernel measured
with HIP events on the launch stream, and the CPU oracle timed on a bounded
sample of the same workload.  The other workloads (bf16 4096^3, skinny
32 x 8192 x 8192, fp8 8192^3) are measured too and reported under "also".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense peaks (TFLOP/s; int8: TOP/s)
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "i8": 5000.0, "w4a8": 5000.0}
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_8192_preshuffled"
# Workloads with fewer 256 x 256 tiles than CUs: timed through gemm_run_ws
# (split K with a workspace), plain gemm_run reported beside.
SPLIT_K_WORKLOADS = ("bf16_256x8192x8192_preshuffled", "bf16_1024x8192x8192", "e4m3_1024x8192x8192",
                     "w4a8_256x8192x8192")
# HBM bytes per launch of the headline kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE scaled by a copy of known size (see the file for the commands).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_pipe_bf16_8192_preshuffled.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_gemm(torch, tg, w, inp, steps, warmup, rotate=1, epi=None, ws=False):
    """Time `steps` gemm_run launches (after `warmup`) with HIP events on the
    launch stream.  With rotate > 1, that many independent input/output sets
    are cycled so the operands are not served from the last-level cache.
    With epi (an epilogue name), gemm_run_ex is timed instead, with per-row
    and per-column scale vectors and a bias vector.  Integer workloads run
    through gemm_run_ex with their per-row / per-channel dequantisation
    scales.  With ws, gemm_run_ws with a workspace of gemm_workspace_bytes
    (split K where the plan splits)."""
    code = {("bf16", "f32"): tg.GEMM_BF16_OUT_F32, ("bf16", "bf16"): tg.GEMM_BF16_OUT_BF16,
            ("e4m3", "bf16"): tg.GEMM_E4M3_OUT_BF16, ("mxfp8", "bf16"): tg.GEMM_MXFP8_OUT_BF16,
            ("mxfp4", "bf16"): tg.GEMM_MXFP4_OUT_BF16, ("i8", "bf16"): tg.GEMM_I8_OUT_BF16,
            ("w4a8", "bf16"): tg.GEMM_W4A8_OUT_BF16}[(w.dtype, w.out)]
    plan = tg.Plan(w.M, w.N, w.K, code, tg.LAYOUTS[w.layout])
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def dev(bits):
        bits = np.ascontiguousarray(bits)
        return torch.from_numpy(bits.view(np.int16) if bits.dtype == np.uint16 else bits).cuda()

    A0, B0 = dev(inp.A), dev(inp.B)
    sets = []
    shuf_ms = None
    for r in range(rotate):
        A = A0 if r == 0 else A0.clone()
        B = B0 if r == 0 else B0.clone()
        if w.layout == "bt_preshuffled":
            Bs = torch.empty(tg.gemm_preshuffled_b_bytes(plan.handle), dtype=torch.uint8, device="cuda")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            plan.preshuffle_b(B.data_ptr(), Bs.data_ptr(), s)      # warm
            e0.record(stream)
            plan.preshuffle_b(B.data_ptr(), Bs.data_ptr(), s)
            e1.record(stream)
            torch.cuda.synchronize()
            shuf_ms = e0.elapsed_time(e1)
            B = Bs
        C = torch.empty(w.M * w.N * w.out_bytes, dtype=torch.uint8, device="cuda")
        sets.append((A, B, C))
    scale = torch.tensor([inp.scale_a, inp.scale_b], dtype=torch.float32, device="cuda")
    sp = scale.data_ptr() if w.dtype == "e4m3" else None
    if w.dtype.startswith("mx"):
        imgs = []
        for operand, blocks in ((0, inp.sa_blocks), (1, inp.sb_blocks)):
            src = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
            img = torch.empty(plan.bscale_image_bytes(operand), dtype=torch.uint8, device="cuda")
            plan.preshuffle_bscale(operand, src.data_ptr(), img.data_ptr(), s)
            imgs.append(img)

        def launch(A, B, C):
            plan.run_mx(A.data_ptr(), imgs[0].data_ptr(), B.data_ptr(), imgs[1].data_ptr(), C.data_ptr(), stream=s)
    elif w.dtype in ("i8", "w4a8"):
        qa = torch.from_numpy(inp.sa_rows).cuda()
        qb = torch.from_numpy(inp.sb_cols).cuda()

        wsb = plan.workspace_bytes() if ws else 0
        Wk = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")

        def launch(A, B, C):
            if ws:
                plan.run_ws(A.data_ptr(), B.data_ptr(), C.data_ptr(), Wk.data_ptr(), wsb, stream=s,
                            scale_a=qa.data_ptr(), scale_a_per_row=True, scale_b=qb.data_ptr(), scale_b_per_col=True)
            else:
                plan.run_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream=s, scale_a=qa.data_ptr(),
                            scale_a_per_row=True, scale_b=qb.data_ptr(), scale_b_per_col=True)
    elif ws:
        wsb = plan.workspace_bytes()
        Wk = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")

        def launch(A, B, C):
            plan.run_ws(A.data_ptr(), B.data_ptr(), C.data_ptr(), Wk.data_ptr(), wsb, stream=s,
                        scale_a=sp, scale_b=sp + 4 if sp else None)
    elif epi is None:
        def launch(A, B, C):
            plan.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), sp, s)
    else:
        g = torch.Generator(device="cpu").manual_seed(w.seed)
        sa = (torch.rand(w.M, generator=g) * 0.04 + 0.01).cuda()
        sb = (torch.rand(w.N, generator=g) * 1.5 + 0.5).cuda()
        bias = torch.randn(w.N, generator=g).cuda()

        def launch(A, B, C):
            plan.run_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream=s, scale_a=sa.data_ptr(),
                        scale_a_per_row=True, scale_b=sb.data_ptr(), scale_b_per_col=True,
                        bias=bias.data_ptr(), epilogue=tg.EPILOGUES[epi])
    for i in range(warmup):
        A, B, C = sets[i % rotate]
        launch(A, B, C)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        A, B, C = sets[i % rotate]
        launch(A, B, C)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    info = plan.info()
    plan.close()
    del sets
    torch.cuda.empty_cache()
    return ms, wall, info, shuf_ms


def cpu_baseline(w, inp, target_s=12.0):
    """The oracle on a bounded sample of the same workload: whole rows of C,
    as many as fit ~target_s seconds (calibrated on a small first sample)."""
    import oracle
    threads = oracle.threads()
    rng = np.random.default_rng(w.seed)

    def run(nrows):
        rows = np.repeat(rng.choice(w.M, size=nrows, replace=False), w.N)
        cols = np.tile(np.arange(w.N), nrows)
        sigma = oracle.sigma_of(inp.scale_a, inp.scale_b)
        t0 = time.perf_counter()
        oracle.gemm_bt_entries(inp.A, inp.B, rows, cols, dtype=w.dtype, sigma=sigma)
        return time.perf_counter() - t0

    probe_rows = max(1, threads // 2)
    t = run(probe_rows)
    nrows = int(max(1, min(w.M, probe_rows * target_s / max(t, 1e-3))))
    t = run(nrows)
    flops = 2.0 * nrows * w.N * w.K
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d full rows of C (%d x %d outputs, K=%d) of %s in %.1f s" % (
                nrows, nrows, w.N, w.K, w.name, t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--only", default=None, help="time only this workload (profiling runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a device-to-device copy of MIB MiB (3 times): the reference "
                         "kernel whose FETCH_SIZE / WRITE_SIZE scale the GEMM's HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only (--gpus %d requested); "
              "the sharded design is described in DESIGN.md" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_gemm_amd as tg
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    tg.load()
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copy calibration %d MiB x 3" % args.calibrate_copy)
        del src, dst
    names = [args.only] if args.only else [HEADLINE] + ([] if args.no_also else [
        "bf16_4096", "bf16_4096_bn", "bf16_4096_at", "bf16_4096_at_bn", "bf16_skinny_32x8192x8192",
        "bf16_skinny_32x8192x8192_preshuffled", "bf16_256x8192x8192_preshuffled", "bf16_1024x8192x8192",
        "e4m3_1024x8192x8192", "e4m3_8192", "e4m3_8192_bn", "mxfp8_8192", "mxfp4_8192", "mxfp4_32x8192x8192",
        "i8_8192", "w4a8_8192", "w4a8_32x8192x8192", "w4a8_256x8192x8192"])
    results = {}
    inputs = {}
    for name in names:
        w = W.WORKLOADS[name]
        log("bench: generating", name)
        inp = W.make_inputs(w)
        rotate = 3 if name.startswith("bf16_skinny_32x8192x8192") or name in ("w4a8_32x8192x8192",
                                                                               "mxfp4_32x8192x8192") else 1
        steps = args.steps if name == (args.only or HEADLINE) else max(10, args.steps // 2)
        split = name in SPLIT_K_WORKLOADS
        if split:
            # split K through gemm_run_ws; the plain gemm_run figure beside it
            ms1, _, _, _ = time_gemm(torch, tg, w, inp, steps, args.warmup, rotate)
        ms, wall, info, shuf_ms = time_gemm(torch, tg, w, inp, steps, args.warmup, rotate, ws=split)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = w.min_bytes / (ms * 1e-3) / 1e9
        results[name] = dict(ms=ms, wall=wall, steps=steps, tflops=tflops, gbs=gbs, info=info,
                             shuf_ms=shuf_ms, rotate=rotate)
        if split:
            results[name]["ms_gemm_run"] = ms1
        log("bench: %-26s %.4f ms  %.1f TFLOP/s  %.0f GB/s  tile %dx%d grid %d" % (
            name, ms, tflops, gbs, info["tile_m"], info["tile_n"], info["grid"]))
        if name == HEADLINE:
            inputs[name] = inp
    if not args.only and not args.no_also:
        # the headline shape again with the fused epilogue: per-row and
        # per-column scales, bias and GELU
        w = W.WORKLOADS[HEADLINE]
        name = HEADLINE + "+scales+bias_gelu"
        ms, wall, info, _ = time_gemm(torch, tg, w, inputs[HEADLINE], max(10, args.steps // 2), args.warmup,
                                      1, epi="bias_gelu")
        results[name] = dict(ms=ms, wall=wall, steps=max(10, args.steps // 2), tflops=w.flops / (ms * 1e-3) / 1e12,
                             gbs=w.min_bytes / (ms * 1e-3) / 1e9, info=info, shuf_ms=None, rotate=1)
        log("bench: %-26s %.4f ms  %.1f TFLOP/s" % (name, ms, results[name]["tflops"]))

    head = args.only or HEADLINE
    w = W.WORKLOADS[head]
    r = results[head]
    # the roofline that bounds the workload: HBM below the ridge point
    # (peak flops / peak HBM bytes per second), MFMA above it
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if w.flops / w.min_bytes < ridge else "mfma"
    traffic = None
    if head == HEADLINE:
        from profile_summary import read_traffic
        traffic = read_traffic(TRAFFIC_FILE)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAK_TFLOPS[w.dtype], 4),
                "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(r["gbs"] / PEAK_HBM_GBS, 4), "traffic": None}
    line = {
        "metric": "GEMM TFLOP/s (bf16 8192^3, B pre-shuffled, fp32 accumulate, bf16 out)",
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp8_e4m3",
        "data": "synthetic (seeded %s)" % w.name,
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": w.layout,
                   "out": w.out, "tile": "%dx%d" % (r["info"]["tile_m"], r["info"]["tile_n"]),
                   "grid": r["info"]["grid"], "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if r["shuf_ms"] is not None:
        line["preshuffle"] = {"ms": round(r["shuf_ms"], 4),
                              "GB/s": round(2 * w.N * w.K * w.b_elem_bytes / (r["shuf_ms"] * 1e-3) / 1e9, 1)}
    also = {}
    for name, rr in results.items():
        if name == head:
            continue
        ww = W.WORKLOADS[name.split("+")[0]]
        also[name] = {"ms": round(rr["ms"], 5), ("TOP/s" if ww.dtype in ("i8", "w4a8") else "TFLOP/s"): round(rr["tflops"], 2),
                      "frac_mfma_peak": round(rr["tflops"] / PEAK_TFLOPS[ww.dtype], 4),
                      "GB/s": round(rr["gbs"], 1), "frac_hbm_peak": round(rr["gbs"] / PEAK_HBM_GBS, 4),
                      "tile": "%dx%d" % (rr["info"]["tile_m"], rr["info"]["tile_n"]),
                      "input_sets_rotated": rr["rotate"]}
        if "ms_gemm_run" in rr:
            # gemm_run_ws: 256 x 256 tiles, K split (the plain gemm_run's own tile may differ)
            also[name]["tile"] = "256x256" if rr["info"]["ws_splits"] > 1 else also[name]["tile"]
            also[name]["split_k"] = rr["info"]["ws_splits"]
            also[name]["ms_gemm_run"] = round(rr["ms_gemm_run"], 5)
    if head in SPLIT_K_WORKLOADS:
        if r["info"]["ws_splits"] > 1:
            line["config"]["tile"] = "256x256"
            line["config"]["grid"] = r["info"]["ws_grid"]
        line["config"]["split_k"] = r["info"]["ws_splits"]
        line["config"]["ms_gemm_run"] = round(r["ms_gemm_run"], 5)
    if also:
        line["also"] = also
    if not args.no_cpu_baseline and head in inputs:
        log("bench: timing the CPU oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(w, inputs[head])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
