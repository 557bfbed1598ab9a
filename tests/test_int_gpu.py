"""Parity of the integer GEMMs (int8 x int8 and W4A8: int8 x packed int4)
with the oracle's exact integer sums.

* Full-range inputs (int8 -128..127, int4 -8..7) whose sums stay below 2^24,
  so fp32 holds them exactly: the bf16 C must match the oracle bit for bit on
  both kernels (8 waves, 4 waves), both layouts, with a half-filled last K
  step (int8), with M and N tails, and through a fused epilogue with
  power-of-two scales and integer bias.
* The extremes: every product at -128 * -128 (int8) or -128 * -8 (int4).
* Quantised N(0,1) inputs with per-row / per-channel scales and SiLU / GELU:
  within the epilogue bound; the full-size workloads on sampled entries.
"""
import numpy as np
import pytest
import torch

import tiled_gemm_amd as tg
import workloads as W
import gpu_util
from gpu_util import assert_epilogue_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu

FMTS = ["i8", "w4a8"]
WAVES = [None, "4"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


def set_waves(monkeypatch, waves):
    # None: the planner's 8-wave kernel; "4": the 4-wave AGPR form.
    gpu_util.force("pipe4" if waves == "4" else None)


def _k_for(fmt, ragged):
    # int8 ragged: K an odd multiple of 64, so the last 128-byte step is half
    # full; W4A8 needs K % 128 == 0, so "ragged" is an odd number of steps
    if fmt == "i8":
        return 1088 if ragged else 1024
    return 1152 if ragged else 1024


def _bits_equal(bits, want, ref):
    bad = bits != want
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])], ref[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("waves", WAVES)
def test_int_bit_exact(oracle_mod, monkeypatch, fmt, layout, ragged, waves):
    M, N, K = 300, 272, _k_for(fmt, ragged)
    set_waves(monkeypatch, waves)
    say("case int exact", fmt, layout, waves, M, N, K)
    inp = W.int_inputs(M, N, K, fmt, seed=K + len(layout), lo=-128, hi=127)
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, return_plan_info=True)
    assert info["b_elem_bits"] == (8 if fmt == "i8" else 4)
    assert info["threads"] == (256 if waves else 512)
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    assert S.max() < 2.0 ** 24            # every sum exact in fp32: one rounding, to bf16
    _bits_equal(bits, oracle_mod.round_bf16(acc), acc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("waves", WAVES)
def test_int_with_epilogue_bit_exact(oracle_mod, monkeypatch, fmt, waves):
    M, N, K = 300, 272, _k_for(fmt, True)
    set_waves(monkeypatch, waves)
    say("case int epilogue exact", fmt, waves, M, N, K)
    inp = W.int_inputs(M, N, K, fmt, seed=77, lo=-128, hi=127)
    rng = np.random.default_rng(5)
    e = dict(scale_a=2.0 ** rng.integers(-8, -2, M), scale_b=-(2.0 ** rng.integers(-3, 3, N)),
             bias=rng.integers(-64, 65, N).astype(np.float64), kind="bias_relu")
    bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", "bt_preshuffled", epi=e)
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    # |acc| < 2^22: acc * 2^e plus an integer bias needs at most ~21 significant
    # bits, so every fp32 step is exact and C is one rounding of the exact value
    assert np.abs(acc).max() < 2.0 ** 22
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e["bias"], e["kind"])
    _bits_equal(bits, oracle_mod.round_bf16(want), want)


# Decode shapes (M <= 64) run on the skinny kernels: int8 with B N x K or
# pre-shuffled, W4A8 with B pre-shuffled.
SKINNY = [("i8", "bt"), ("i8", "bt_preshuffled"), ("w4a8", "bt_preshuffled")]


@pytest.mark.parametrize("fmt,layout", SKINNY)
@pytest.mark.parametrize("M", [1, 17, 32, 33, 64])
@pytest.mark.parametrize("N", [544, 528])
def test_int_skinny_bit_exact(oracle_mod, fmt, layout, M, N):
    K = _k_for(fmt, True)
    say("case int skinny exact", fmt, layout, M, N, K)
    inp = W.int_inputs(M, N, K, fmt, seed=M + N, lo=-128, hi=127)
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, return_plan_info=True)
    assert info["kernel"] == 1
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    assert S.max() < 2.0 ** 24
    _bits_equal(bits, oracle_mod.round_bf16(acc), acc)


@pytest.mark.parametrize("fmt,layout", SKINNY)
def test_int_skinny_large_sums_exact_in_int32(oracle_mod, fmt, layout):
    # every product at its extreme over K = 8192: the waves' partial sums are
    # combined in int32, so the one rounding is the final one
    M, N, K = 32, 544, 8192
    say("case int skinny extremes", fmt, layout)
    A = np.full((M, K), 0x80, np.uint8)
    B = np.full((N, K), 0x80, np.uint8) if fmt == "i8" else np.full((N, K // 2), 0x88, np.uint8)
    bits = run_gemm(A, B, M, N, K, fmt, "bf16", layout)
    acc, _ = oracle_mod.gemm_bt_int_entries(A, B, K, [0], [0], fmt)
    assert acc[0] == (2.0 ** 27 if fmt == "i8" else 2.0 ** 23)
    assert np.all(bits == oracle_mod.round_bf16(acc)[0])


@pytest.mark.parametrize("fmt,layout", SKINNY)
@pytest.mark.parametrize("kind", ["none", "bias_gelu"])
def test_int_skinny_quantised_within_bound(oracle_mod, fmt, layout, kind):
    M, N, K = 32, 784, 1536
    say("case int skinny quantised", fmt, layout, kind)
    inp = W.make_inputs(W.WORKLOADS[fmt + "_8192"], M=M, N=N, K=K, seed=41)
    rng = np.random.default_rng(42)
    e = dict(scale_a=inp.sa_rows.astype(np.float64), scale_b=inp.sb_cols.astype(np.float64), kind=kind)
    if kind != "none":
        e["bias"] = rng.normal(0.0, 1.0, N)
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, epi=e, return_plan_info=True)
    assert info["kernel"] == 1
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e.get("bias"), kind)
    scale = np.abs(e["scale_a"][:, None] * e["scale_b"][None, :])
    bias_abs = np.abs(e["bias"])[None, :] if "bias" in e else 0.0
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale, bias_abs, fmt, kind,
                                     "skinny %s %s" % (fmt, kind))
    say("  worst err/bound", r)


def test_w4a8_plain_decode_stays_tiled():
    # W4A8 with B N x K (packed rows) has no skinny kernel
    with tg.Plan(32, 8192, 8192, tg.GEMM_W4A8_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert p.info()["kernel"] == 0


@pytest.mark.parametrize("fmt", FMTS)
def test_int_extremes(oracle_mod, fmt):
    # every product at its largest magnitude: -128 * -128 = 2^14 (int8) or
    # -128 * -8 = 2^10 (int4), summed over K = 16384: 2^28 or 2^24
    M, N, K = 256, 256, 16384
    say("case int extremes", fmt, M, N, K)
    A = np.full((M, K), 0x80, np.uint8)
    B = np.full((N, K), 0x80, np.uint8) if fmt == "i8" else np.full((N, K // 2), 0x88, np.uint8)
    bits = run_gemm(A, B, M, N, K, fmt, "bf16", "bt")
    acc, _ = oracle_mod.gemm_bt_int_entries(A, B, K, [0], [0], fmt)
    assert acc[0] == (2.0 ** 28 if fmt == "i8" else 2.0 ** 24)
    assert np.all(bits == oracle_mod.round_bf16(acc)[0])


@pytest.mark.parametrize("fmt", FMTS)
def test_int_k_zero_and_tiny(oracle_mod, fmt):
    say("case int K=0", fmt)
    bits = run_gemm(np.zeros((40, 0), np.uint8), np.zeros((32, 0), np.uint8), 40, 32, 0, fmt, "bf16", "bt",
                    epi=dict(scale_a=2.0, bias=np.arange(32, dtype=np.float64), kind="bias"))
    assert np.array_equal(decode(bits), np.tile(np.arange(32, dtype=np.float64), (40, 1)))
    M, N, K = 1, 16, 128
    say("case int tiny", fmt, M, N, K)
    inp = W.int_inputs(M, N, K, fmt, seed=3, lo=-128, hi=127)
    for layout in ("bt", "bt_preshuffled"):
        bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout)
        acc, _ = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
        _bits_equal(bits, oracle_mod.round_bf16(acc), acc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["none", "bias_silu", "bias_gelu"])
@pytest.mark.parametrize("waves", WAVES)
def test_int_quantised_within_bound(oracle_mod, monkeypatch, fmt, kind, waves):
    M, N, K = 520, 784, 1536
    set_waves(monkeypatch, waves)
    say("case int quantised", fmt, kind, waves, M, N, K)
    inp = W.make_inputs(W.WORKLOADS[fmt + "_8192"], M=M, N=N, K=K, seed=31)
    rng = np.random.default_rng(32)
    e = dict(scale_a=inp.sa_rows.astype(np.float64), scale_b=inp.sb_cols.astype(np.float64), kind=kind)
    if kind != "none":
        e["bias"] = rng.normal(0.0, 1.0, N)
    bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", "bt_preshuffled", epi=e)
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, fmt)
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e.get("bias"), kind)
    scale = np.abs(e["scale_a"][:, None] * e["scale_b"][None, :])
    bias_abs = np.abs(e["bias"])[None, :] if "bias" in e else 0.0
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale, bias_abs, fmt, kind,
                                     "%s %s" % (fmt, kind))
    say("  worst err/bound", r)


@pytest.mark.parametrize("name", ["i8_8192", "i8_8192_bt", "w4a8_8192", "w4a8_32x8192x8192"])
def test_int_full_size_sampled(oracle_mod, monkeypatch, name):
    set_waves(monkeypatch, None)
    w = W.WORKLOADS[name]
    say("case int full-size", name)
    inp = W.make_inputs(w)
    e = dict(scale_a=inp.sa_rows.astype(np.float64), scale_b=inp.sb_cols.astype(np.float64), kind="none")
    bits = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout, epi=e)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    acc, S = oracle_mod.gemm_bt_int_entries(inp.A, inp.B, w.K, rows, cols, w.dtype)
    want = oracle_mod.epilogue_entries(acc, e["scale_a"][rows], e["scale_b"][cols], None, "none")
    scale = np.abs(e["scale_a"][rows] * e["scale_b"][cols])
    r = assert_epilogue_within_bound(decode(bits[rows, cols]), want, S * scale, np.abs(acc) * scale, 0.0,
                                     w.dtype, "none", name)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))
