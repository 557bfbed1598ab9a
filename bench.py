"""Benchmark of the tiled GEMM on one MI355X.

A step is one gemm_run of C = A * B^T on the headline workload: bf16
8192 x 8192 x 8192 with B pre-shuffled into MFMA operand order (the
pre-shuffle is done once, ahead of the timed steps, and reported separately),
fp32 accumulation, bf16 output.  Inputs are seeded synthetic data resident in
HBM before timing starts; three independent input/output sets are cycled so
the 256 MB last-level cache does not serve the operands of the launch being
timed.

Timing (HIP events recorded on the launch stream):
  * `sustained` (first): the kernel back to back for a few seconds while the
    GPU clock and socket power are sampled (amd-smi), with the TFLOP/s of
    that stretch: the card runs at its power limit, so the clock it settles
    at is part of the result.  This also brings the GPU out of the idle clock
    state it drops to while the host draws the inputs (the other workloads
    get a short untimed stretch instead);
  * `value` / `ms_per_step`: then W warmup steps and exactly K steps between
    one pair of events (the mean launch duration);
  * `timing`: 50 further launches, each between its own pair of events:
    median and minimum (the pages' do_bench reports the median).
The other workloads (the five configurations of the survey and the next
rows: bf16 4096^3 in every layout, the decode shape, split K, fp8, MX,
int8, W4A8) are measured the same way and reported under "also", the oracle
timed beside the configurations it checks.

Prints one JSON line with TFLOP/s, the roofline of the GEMM kernel and the
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense peaks (TFLOP/s; int8: TOP/s)
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "i8": 5000.0, "w4a8": 5000.0}
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_8192_preshuffled"
# The five configurations the survey names, by workload.
CONFIGS = {"c1": "bf16_int_256", "c2": "bf16_4096", "c3": HEADLINE, "c4": "bf16_skinny_32x8192x8192",
           "c5": "e4m3_8192"}
ALSO = ["bf16_int_256", "bf16_4096", "bf16_4096_bn", "bf16_4096_at", "bf16_4096_at_bn", "bf16_skinny_32x8192x8192",
        "bf16_skinny_32x8192x8192_preshuffled", "bf16_256x8192x8192_preshuffled", "bf16_1024x8192x8192",
        "e4m3_1024x8192x8192", "e4m3_8192", "e4m3_8192_preshuffled", "e4m3_8192_bn", "mxfp8_8192", "mxfp4_8192",
        "mxfp4_32x8192x8192", "i8_8192", "i8_8192_bt", "w4a8_8192", "w4a8_32x8192x8192", "w4a8_256x8192x8192"]
# Workloads with fewer 256 x 256 tiles than CUs: timed through gemm_run_ws
# (split K with a workspace), plain gemm_run reported beside.
SPLIT_K_WORKLOADS = ("bf16_256x8192x8192_preshuffled", "bf16_1024x8192x8192", "e4m3_1024x8192x8192",
                     "w4a8_256x8192x8192")
ROTATE = 3                   # input/output sets cycled through
REPS = 50                    # individually timed launches (median, minimum)
WARM_S = 0.3                 # untimed back-to-back launches before each measurement
# HBM bytes per launch of the headline kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE scaled by a copy of known size (see the file for the commands).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_pipe_bf16_8192_preshuffled.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_clock_sample():
    """(mean GFX clock in MHz over the XCDs, socket power in W) from amd-smi, or None."""
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                             text=True, timeout=30).stdout
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)]
        return float(np.mean(clks)), float(g["power"]["socket_power"]["value"])
    except Exception as e:            # the tool is optional: report no sample
        log("bench: no clock sample (%s)" % (e,))
        return None


class Runner:
    """One workload set up for timing: plan, ROTATE input/output sets in HBM,
    and a launch(i) that runs set i % ROTATE through the entry point the
    workload uses."""

    def __init__(self, torch, tg, w, inp, rotate=ROTATE, epi=None, ws=False):
        self.torch, self.w = torch, w
        code = {("bf16", "f32"): tg.GEMM_BF16_OUT_F32, ("bf16", "bf16"): tg.GEMM_BF16_OUT_BF16,
                ("e4m3", "bf16"): tg.GEMM_E4M3_OUT_BF16, ("mxfp8", "bf16"): tg.GEMM_MXFP8_OUT_BF16,
                ("mxfp4", "bf16"): tg.GEMM_MXFP4_OUT_BF16, ("i8", "bf16"): tg.GEMM_I8_OUT_BF16,
                ("w4a8", "bf16"): tg.GEMM_W4A8_OUT_BF16}[(w.dtype, w.out)]
        self.plan = plan = tg.Plan(w.M, w.N, w.K, code, tg.LAYOUTS[w.layout])
        self.stream = stream = torch.cuda.current_stream()
        s = stream.cuda_stream

        def dev(bits):
            bits = np.ascontiguousarray(bits)
            return torch.from_numpy(bits.view(np.int16) if bits.dtype == np.uint16 else bits).cuda()

        A0, B0 = dev(inp.A), dev(inp.B)
        self.sets = []
        self.shuf_ms = None
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
                self.shuf_ms = e0.elapsed_time(e1)
                B = Bs
            C = torch.empty(w.M * w.N * w.out_bytes, dtype=torch.uint8, device="cuda")
            self.sets.append((A, B, C))
        del A0, B0
        scale = torch.tensor([inp.scale_a, inp.scale_b], dtype=torch.float32, device="cuda")
        self._keep = [scale]
        sp = scale.data_ptr() if w.dtype == "e4m3" else None
        if w.dtype.startswith("mx"):
            imgs = []
            for operand, blocks in ((0, inp.sa_blocks), (1, inp.sb_blocks)):
                src = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
                img = torch.empty(plan.bscale_image_bytes(operand), dtype=torch.uint8, device="cuda")
                plan.preshuffle_bscale(operand, src.data_ptr(), img.data_ptr(), s)
                imgs.append(img)
            self._keep += imgs

            def launch(A, B, C):
                plan.run_mx(A.data_ptr(), imgs[0].data_ptr(), B.data_ptr(), imgs[1].data_ptr(), C.data_ptr(),
                            stream=s)
        elif w.dtype in ("i8", "w4a8"):
            qa = torch.from_numpy(inp.sa_rows).cuda()
            qb = torch.from_numpy(inp.sb_cols).cuda()
            wsb = plan.workspace_bytes() if ws else 0
            Wk = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")
            self._keep += [qa, qb, Wk]

            def launch(A, B, C):
                if ws:
                    plan.run_ws(A.data_ptr(), B.data_ptr(), C.data_ptr(), Wk.data_ptr(), wsb, stream=s,
                                scale_a=qa.data_ptr(), scale_a_per_row=True, scale_b=qb.data_ptr(),
                                scale_b_per_col=True)
                else:
                    plan.run_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream=s, scale_a=qa.data_ptr(),
                                scale_a_per_row=True, scale_b=qb.data_ptr(), scale_b_per_col=True)
        elif ws:
            wsb = plan.workspace_bytes()
            Wk = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")
            self._keep.append(Wk)

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
            self._keep += [sa, sb, bias]

            def launch(A, B, C):
                plan.run_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream=s, scale_a=sa.data_ptr(),
                            scale_a_per_row=True, scale_b=sb.data_ptr(), scale_b_per_col=True,
                            bias=bias.data_ptr(), epilogue=tg.EPILOGUES[epi])
        self._launch = launch
        self.info = plan.info()

    def launch(self, i):
        A, B, C = self.sets[i % len(self.sets)]
        self._launch(A, B, C)

    def timed(self, steps, warmup):
        """W warmup launches, then `steps` launches between one pair of events:
        (mean ms per launch, wall seconds of the timed region)."""
        torch = self.torch
        for i in range(warmup):
            self.launch(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(steps):
            self.launch(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t0

    def reps(self, n=REPS):
        """n launches, each between its own pair of events: sorted ms."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (a, b) in enumerate(ev):
            a.record(self.stream)
            self.launch(i)
            b.record(self.stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    def warm(self, seconds):
        """Launches back to back for about `seconds` (untimed), so that the
        GPU clock has left its idle state before a measurement."""
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(16):
                self.launch(n)
                n += 1
            self.torch.cuda.synchronize()

    def sustained(self, seconds):
        """The kernel back to back for about `seconds` while amd-smi samples the
        GPU clock and socket power.  Returns (TFLOP/s over the stretch, finish):
        finish() stops the sampling and returns the samples.  The caller goes on
        launching before calling it, so that the GPU does not idle (an idle
        stretch of tens of milliseconds drops the clock, and the launches after
        it run up to 30% slower until it recovers)."""
        torch = self.torch
        samples, stop = [], threading.Event()

        def sampler():
            time.sleep(0.5)
            while not stop.is_set():
                s = gpu_clock_sample()
                if s is None:
                    return
                samples.append(s)
        th = threading.Thread(target=sampler, daemon=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        th.start()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(64):
                self.launch(n)
                n += 1
            torch.cuda.synchronize()
        e1.record(self.stream)
        torch.cuda.synchronize()
        stop.set()
        ms = e0.elapsed_time(e1) / n

        def finish():
            th.join(timeout=60)
            return samples
        return self.w.flops / (ms * 1e-3) / 1e12, finish

    def close(self):
        self.plan.close()
        self.sets = []
        self._keep = []
        self.torch.cuda.empty_cache()


def oracle_rate(w, inp, target_s):
    """The oracle on a bounded sample of workload w: whole rows of C, as many
    as fit about target_s seconds (calibrated on a small first sample).
    Returns (flop/s, rows, seconds, threads)."""
    import oracle
    threads = oracle.threads()
    rng = np.random.default_rng(w.seed)
    sigma = oracle.sigma_of(inp.scale_a, inp.scale_b)

    def run(nrows):
        rows = np.repeat(rng.choice(w.M, size=nrows, replace=False), w.N)
        cols = np.tile(np.arange(w.N), nrows)
        t0 = time.perf_counter()
        if w.dtype == "bf16" or w.dtype == "e4m3":
            oracle.gemm_bt_entries(inp.A, inp.B, rows, cols, dtype=w.dtype, sigma=sigma)
        else:
            raise ValueError("oracle timing covers the bf16 and e4m3 configurations")
        return time.perf_counter() - t0

    probe_rows = max(1, min(w.M, threads // 2))
    t = run(probe_rows)
    nrows = int(max(1, min(w.M, probe_rows * target_s / max(t, 1e-3))))
    t = run(nrows)
    return 2.0 * nrows * w.N * w.K / t, nrows, t, threads


def cpu_baseline(w, inp, target_s=12.0):
    """The oracle as it stands, on all host cores, over whole rows of C of the
    headline workload (about target_s seconds of CPU work)."""
    rate, nrows, t, threads = oracle_rate(w, inp, target_s)
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d full rows of C (%d x %d outputs, K=%d) of %s in %.1f s" % (
                nrows, nrows, w.N, w.K, w.name, t)}


def summary(w, ms, reps, info, rotate):
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.min_bytes / (ms * 1e-3) / 1e9
    unit = "TOP/s" if w.dtype in ("i8", "w4a8") else "TFLOP/s"
    med, mn = float(np.median(reps)), float(reps[0])
    return {"ms": round(ms, 5), unit: round(tflops, 2), "frac_mfma_peak": round(tflops / PEAK_TFLOPS[w.dtype], 4),
            "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "median_ms": round(med, 5), "min_ms": round(mn, 5),
            "median_" + unit: round(w.flops / (med * 1e-3) / 1e12, 2),
            "tile": "%dx%d" % (info["tile_m"], info["tile_n"]), "input_sets_rotated": rotate}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--only", default=None,
                    help="time only these workloads (comma-separated; the first is the line's subject)")
    ap.add_argument("--reps", type=int, default=REPS, help="individually timed launches (median, minimum)")
    ap.add_argument("--warm", type=float, default=WARM_S, metavar="SECONDS",
                    help="untimed back-to-back launches before each measurement (0 for profiling runs)")
    ap.add_argument("--sustain", type=float, default=3.0, metavar="SECONDS",
                    help="seconds of back-to-back launches with clock sampling (0: skip)")
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
    only = args.only.split(",") if args.only else None
    head = only[0] if only else HEADLINE
    names = only if only else [head] + ([] if args.no_also else ALSO)
    oracle_for = {v: k for k, v in CONFIGS.items()} if not (only or args.no_cpu_baseline) else {}
    results = {}
    line_extra = {}
    for name in names:
        w = W.WORKLOADS[name]
        log("bench: generating", name)
        inp = W.make_inputs(w)
        is_head = name == head
        steps = args.steps if is_head else max(10, args.steps // 2)
        split = name in SPLIT_K_WORKLOADS
        ms1 = None
        if split:
            # split K through gemm_run_ws; the plain gemm_run figure beside it
            r1 = Runner(torch, tg, w, inp)
            r1.warm(args.warm)
            ms1, _ = r1.timed(steps, args.warmup)
            r1.close()
        run = Runner(torch, tg, w, inp, ws=split)
        # Before the timed steps: the headline's sustained run (clock and power
        # sampled), else a short untimed stretch.  Either takes the GPU out of
        # the idle clock state it drops to while the host draws the inputs.
        finish = None
        if is_head and args.sustain > 0:
            tf, finish = run.sustained(args.sustain)
        else:
            run.warm(args.warm)
        ms, wall = run.timed(steps, args.warmup)
        reps = run.reps(args.reps)
        if finish is not None:
            samples = finish()
            line_extra["sustained"] = {"seconds": args.sustain, "TFLOP/s": round(tf, 2),
                                       "gfx_clock_mhz": [round(s[0]) for s in samples],
                                       "socket_power_w": [round(s[1]) for s in samples]}
            log("bench: sustained %.1f s: %.1f TFLOP/s, clock %s MHz, power %s W" % (
                args.sustain, tf, line_extra["sustained"]["gfx_clock_mhz"],
                line_extra["sustained"]["socket_power_w"]))
        res = summary(w, ms, reps, run.info, ROTATE)
        res["_wall"] = wall
        res["_info"] = run.info
        res["_shuf_ms"] = run.shuf_ms
        res["_steps"] = steps
        if split:
            res["tile"] = "256x256" if run.info["ws_splits"] > 1 else res["tile"]
            res["split_k"] = run.info["ws_splits"]
            res["ms_gemm_run"] = round(ms1, 5)
        run.close()
        if name in oracle_for and not is_head:
            rate, nrows, t, threads = oracle_rate(w, inp, 2.0)
            res["oracle"] = {"GFLOP/s": round(rate / 1e9, 2), "cores": threads,
                             "sample": "%d full rows of C in %.1f s" % (nrows, t)}
        results[name] = res
        log("bench: %-36s %.4f ms (median %.4f, min %.4f)  %.1f TFLOP/s  %.0f GB/s  tile %s" % (
            name, ms, res["median_ms"], res["min_ms"], w.flops / ms / 1e9, res["GB/s"], res["tile"]))
        if is_head:
            head_inp = inp
    if not args.only and not args.no_also:
        # the headline shape again with the fused epilogue: per-row and
        # per-column scales, bias and GELU
        w = W.WORKLOADS[HEADLINE]
        run = Runner(torch, tg, w, head_inp, epi="bias_gelu")
        run.warm(args.warm)
        steps = max(10, args.steps // 2)
        ms, wall = run.timed(steps, args.warmup)
        res = summary(w, ms, run.reps(args.reps), run.info, ROTATE)
        run.close()
        results[HEADLINE + "+scales+bias_gelu"] = res
        log("bench: %-36s %.4f ms  %.1f TFLOP/s" % (HEADLINE + "+scales+bias_gelu", ms, w.flops / ms / 1e9))

    w = W.WORKLOADS[head]
    r = results[head]
    tflops = w.flops / (r["ms"] * 1e-3) / 1e12
    gbs = w.min_bytes / (r["ms"] * 1e-3) / 1e9
    # the roofline that bounds the workload: HBM below the ridge point
    # (peak flops / peak HBM bytes per second), MFMA above it
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if w.flops / w.min_bytes < ridge else "mfma"
    traffic = None
    if head == HEADLINE:
        from profile_summary import read_traffic
        traffic = read_traffic(TRAFFIC_FILE)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS[w.dtype], 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    line = {
        "metric": "GEMM TFLOP/s (bf16 8192^3, B pre-shuffled, fp32 accumulate, bf16 out)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": r["_steps"],
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "e4m3": "fp8_e4m3"}.get(w.dtype, w.dtype),
        "data": "synthetic (seeded %s, %d input sets rotated)" % (w.name, ROTATE),
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": w.layout,
                   "out": w.out, "tile": r["tile"], "grid": r["_info"]["grid"], "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": None,
        "timing": {"reps": args.reps, "median_ms": r["median_ms"], "min_ms": r["min_ms"],
                   "median_TFLOP/s": round(w.flops / (r["median_ms"] * 1e-3) / 1e12, 2),
                   "max_TFLOP/s": round(w.flops / (r["min_ms"] * 1e-3) / 1e12, 2)},
    }
    line.update(line_extra)
    if r["_shuf_ms"] is not None:
        line["preshuffle"] = {"ms": round(r["_shuf_ms"], 4),
                              "GB/s": round(2 * w.N * w.K * w.b_elem_bytes / (r["_shuf_ms"] * 1e-3) / 1e9, 1)}
    if head in SPLIT_K_WORKLOADS:
        if r["_info"]["ws_splits"] > 1:
            line["config"]["tile"] = "256x256"
            line["config"]["grid"] = r["_info"]["ws_grid"]
        line["config"]["split_k"] = r["_info"]["ws_splits"]
        line["config"]["ms_gemm_run"] = r["ms_gemm_run"]
    also = {n: {k: v for k, v in rr.items() if not k.startswith("_")} for n, rr in results.items() if n != head}
    if also:
        line["also"] = also
        line["configs"] = CONFIGS
    if not args.no_cpu_baseline and head == HEADLINE:
        log("bench: timing the CPU oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(w, head_inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
