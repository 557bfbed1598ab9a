"""GPU parity of the split-K path (gemm_run_ws) against the CPU oracle.

Split K divides each 256 x 256 tile's K range among several workgroups that
write fp32 partials into the caller's workspace; a second kernel sums them in
slice order and applies the epilogue.  Integer-valued inputs keep every
partial and every sum exact in fp32, so those cases are bit-exact whatever the
slicing; random inputs are held to the GEMM error bound; the full-size case
is checked on sampled entries.
"""
import sys

import numpy as np
import pytest
import torch

import tiled_gemm_amd as tg
import workloads as W
import gpu_util
from gpu_util import assert_epilogue_within_bound, assert_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu

CODES = {("bf16", "f32"): tg.GEMM_BF16_OUT_F32, ("bf16", "bf16"): tg.GEMM_BF16_OUT_BF16,
         ("e4m3", "bf16"): tg.GEMM_E4M3_OUT_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def splits_of(M, N, K, dtype, out, layout):
    with gpu_util.plan(M, N, K, CODES[(dtype, out)], tg.LAYOUTS[layout]) as p:
        return p.info()["ws_splits"]


def exact(oracle_mod, inp, M, N, K, dtype, out, layout, scale=(1.0, 1.0), **kw):
    bits = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, scale=scale, **kw)
    C_ref, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype, sigma=oracle_mod.sigma_of(*scale), want_s=False)
    want = C_ref.astype(np.float32).view(np.uint32) if out == "f32" else oracle_mod.round_bf16(C_ref)
    bad = np.argwhere(bits != want)
    assert bad.size == 0, "%d mismatches, first %s: got %s want %s" % (
        len(bad), bad[:3].tolist(), hex(bits[tuple(bad[0])]), hex(want[tuple(bad[0])]))
    return bits


# K = 4160: 65 steps of 128 bytes, the last one half full; integer sums stay
# below 2^24.  N = 784 leaves a ragged last column tile.
@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M", [65, 200, 300, 520])
def test_split_integer_exact(oracle_mod, layout, out, M):
    N, K = 784, 4160
    s = splits_of(M, N, K, "bf16", out, layout)
    say("case split int-exact", layout, out, M, N, K, "splits", s)
    assert s > 1
    inp = W.int_inputs(M, N, K, "bf16", seed=M + 5)
    exact(oracle_mod, inp, M, N, K, "bf16", out, layout, workspace=True)


@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("M", [65, 300])
def test_split_fp8_exact(oracle_mod, monkeypatch, layout, M):
    # e4m3 integers in [-4, 4], per-tensor scales 0.5 and 0.25 (applied by the
    # reduction); K = 4160 bytes: 33 steps, the last one half full.  At these
    # sizes the planner keeps fp8 unsplit, so the split is forced.
    gpu_util.force(splits=4)
    N, K = 784, 4160
    s = splits_of(M, N, K, "e4m3", "bf16", layout)
    say("case split fp8 exact", layout, M, "splits", s)
    assert s > 1
    inp = W.int_inputs(M, N, K, "e4m3", seed=M + 9)
    exact(oracle_mod, inp, M, N, K, "e4m3", "bf16", layout, scale=(0.5, 0.25), workspace=True)


def test_split_fp8_random_within_bound(oracle_mod, monkeypatch):
    gpu_util.force(splits=3)
    M, N, K = 200, 784, 4160
    inp = W.make_inputs(W.WORKLOADS["e4m3_8192"], M=M, N=N, K=K, seed=4444)
    bits = run_gemm(inp.A, inp.B, M, N, K, "e4m3", "bf16", "bt_preshuffled", scale=(inp.scale_a, inp.scale_b),
                    workspace=True)
    C_ref, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype="e4m3", sigma=oracle_mod.sigma_of(inp.scale_a, inp.scale_b))
    r = assert_within_bound(decode(bits), C_ref, S, "e4m3", "split fp8 random")
    say("  worst err/bound", r)


@pytest.mark.parametrize("fmt,layout", [("i8", "bt"), ("i8", "bt_preshuffled"), ("w4a8", "bt"),
                                        ("w4a8", "bt_preshuffled")])
@pytest.mark.parametrize("M", [65, 300])
def test_split_int_exact(oracle_mod, monkeypatch, fmt, layout, M):
    # full-range int8 / int4 values with sums below 2^24: the partials, their
    # sum and the one rounding to bf16 are exact; per-row / per-column
    # power-of-two dequantisation scales in the reduction's epilogue.  K =
    # 2048 keeps every sum of |a b| below 2^24 (16 steps: two slices, forced,
    # since the planner keeps the partials within B's bytes).
    gpu_util.force(splits=2)
    N, K = 784, 2048
    with gpu_util.plan(M, N, K, tg.GEMM_I8_OUT_BF16 if fmt == "i8" else tg.GEMM_W4A8_OUT_BF16, tg.LAYOUTS[layout]) as p:
        s = p.info()["ws_splits"]
    say("case split int exact", fmt, layout, M, "splits", s)
    assert s > 1
    inp = W.int_inputs(M, N, K, fmt, seed=M + len(layout), lo=-128, hi=127)
    rng = np.random.default_rng(M)
    e = dict(scale_a=2.0 ** rng.integers(-3, 1, M), scale_b=2.0 ** rng.integers(-3, 1, N), kind="none")
    bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, epi=e, workspace=True)
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    assert S.max() < 2.0 ** 24
    want = oracle_mod.round_bf16(oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], None, "none"))
    bad = np.argwhere(bits != want)
    assert bad.size == 0, "%d mismatches, first %s" % (len(bad), bad[:3].tolist())


@pytest.mark.parametrize("splits", [2, 3, 5, 8])
def test_split_forced_counts(oracle_mod, monkeypatch, splits):
    # uneven slices (65 steps over 3 or 5 slices), every slice non-empty
    gpu_util.force(splits=splits)
    M, N, K = 136, 528, 4160
    assert splits_of(M, N, K, "bf16", "bf16", "bt_preshuffled") == splits
    say("case split forced", splits)
    inp = W.int_inputs(M, N, K, "bf16", seed=splits)
    exact(oracle_mod, inp, M, N, K, "bf16", "bf16", "bt_preshuffled", workspace=True)


@pytest.mark.parametrize("ws", ["none", "short"])
def test_no_or_short_workspace_runs_unsplit(oracle_mod, ws):
    M, N, K = 200, 784, 4160
    inp = W.int_inputs(M, N, K, "bf16", seed=11)
    with tg.Plan(M, N, K, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        need = p.workspace_bytes()
    assert need > 0
    say("case split fallback", ws, need)
    exact(oracle_mod, inp, M, N, K, "bf16", "bf16", "bt", workspace=0 if ws == "none" else need - 16)


def test_split_repeat_bitwise_stable():
    M, N, K = 256, 1024, 8192
    w = W.WORKLOADS["bf16_8192_preshuffled"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=31)
    a = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", "bt_preshuffled", workspace=True)
    b = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", "bt_preshuffled", workspace=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_split_random_within_bound(oracle_mod, layout, out):
    M, N, K = 200, 784, 4160
    w = W.WORKLOADS["bf16_4096"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=4343)
    say("case split random", layout, out)
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", out, layout, workspace=True)
    C_ref, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype="bf16")
    r = assert_within_bound(decode(bits), C_ref, S, "bf16", "split random %s %s" % (layout, out))
    say("  worst err/bound", r)


@pytest.mark.parametrize("kind", ["bias", "bias_relu"])
def test_split_epilogue_exact(oracle_mod, kind):
    M, N, K = 300, 528, 4160
    rng = np.random.default_rng(3)
    p2 = lambda n: (2.0 ** rng.integers(-2, 3, n)) * rng.choice([-1.0, 1.0], n)
    e = dict(scale_a=p2(M), scale_b=p2(N), bias=rng.integers(-8, 9, N).astype(np.float64), kind=kind)
    inp = W.int_inputs(M, N, K, "bf16", seed=17)
    say("case split epilogue exact", kind)
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "f32", "bt", epi=e, workspace=True)
    acc, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype="bf16")
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e["bias"], kind)
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want)
    assert np.array_equal(bits, want.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("kind", ["bias_silu", "bias_gelu"])
def test_split_epilogue_smooth(oracle_mod, kind):
    M, N, K = 200, 784, 4160
    w = W.WORKLOADS["bf16_4096"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=99)
    rng = np.random.default_rng(100)
    sa = rng.uniform(0.02, 0.1, M)
    sb = rng.uniform(0.5, 2.0, N)
    e = dict(scale_a=sa, scale_b=sb, bias=rng.normal(0.0, 1.0, N), kind=kind)
    say("case split epilogue smooth", kind)
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", "bt_preshuffled", epi=e, workspace=True)
    acc, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype="bf16")
    want = oracle_mod.epilogue(acc, sa, sb, e["bias"], kind)
    scale = np.abs(sa[:, None] * sb[None, :])
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"])[None, :], "bf16", kind, "split " + kind)
    say("  worst err/bound", r)


@pytest.mark.parametrize("name", ["bf16_256x8192x8192_preshuffled", "bf16_1024x8192x8192", "e4m3_1024x8192x8192",
                                  "w4a8_256x8192x8192"])
def test_split_full_size_sampled(oracle_mod, name):
    w = W.WORKLOADS[name]
    say("case split full-size", name)
    inp = W.make_inputs(w)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    if w.dtype in ("i8", "w4a8"):
        e = dict(scale_a=inp.sa_rows.astype(np.float64), scale_b=inp.sb_cols.astype(np.float64), kind="none")
        bits, info = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout, epi=e, workspace=True,
                              return_plan_info=True)
        acc, s = oracle_mod.gemm_bt_int_entries(inp.A, inp.B, w.K, rows, cols, w.dtype)
        scale = np.abs(e["scale_a"][rows] * e["scale_b"][cols])
        c_ref = oracle_mod.epilogue_entries(acc, e["scale_a"][rows], e["scale_b"][cols], None, "none")
        r = assert_epilogue_within_bound(decode(bits[rows, cols]), c_ref, s * scale, np.abs(acc) * scale, 0.0,
                                         w.dtype, "none", name)
    else:
        bits, info = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout, workspace=True,
                              scale=(inp.scale_a, inp.scale_b), return_plan_info=True)
        c_ref, s = oracle_mod.gemm_bt_entries(inp.A, inp.B, rows, cols, dtype=w.dtype,
                                              sigma=oracle_mod.sigma_of(inp.scale_a, inp.scale_b))
        r = assert_within_bound(decode(bits[rows, cols]), c_ref, s, w.dtype, name)
    say("  plan", info)
    assert info["ws_splits"] > 1
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))
