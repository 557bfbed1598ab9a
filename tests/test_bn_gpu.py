"""Parity of C = A * B with B stored K x N (GEMM_LAYOUT_BN, read through
the LDS transpose load) with the oracle's gemm_ab, for bf16 and fp8 e4m3.

* Integer-valued bf16 inputs (exact sums): bit-exact on both tile sizes and
  both outputs, with M and N tails, a half-filled last K step (K % 64 ==
  32) and the smallest shapes.
* N(0,1) inputs: within the GEMM bound; the 4096^3 workload on sampled
  entries; a fused epilogue.
"""
import numpy as np
import pytest
import torch

import workloads as W
import gpu_util
from gpu_util import assert_epilogue_within_bound, assert_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


def set_tile(monkeypatch, tile):
    # "tile256": the planner's 256 x 256 kernel (both operands staged in LDS);
    # "generic256" / "generic128": the generic tiled kernel.
    gpu_util.force(tile)


def int_kn(M, N, K, seed):
    """Integer-valued bf16 A (M x K) and B stored K x N."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-4, 5, (M, K)).astype(np.float32)
    b = rng.integers(-4, 5, (K, N)).astype(np.float32)
    return W.to_bf16_bits(a), W.to_bf16_bits(b)


def _exact(oracle_mod, bits, out, C):
    if out == "f32":
        want = C.astype(np.float32).view(np.uint32)
    else:
        want = oracle_mod.round_bf16(C)
    bad = bits != want
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])], C[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("tile", ["tile256", "generic256", "generic128"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 272, 1056), (256, 512, 1024), (1, 16, 32), (77, 48, 96)])
def test_bn_bit_exact(oracle_mod, monkeypatch, tile, out, M, N, K):
    set_tile(monkeypatch, tile)
    say("case bn exact", tile, out, M, N, K)
    A, B = int_kn(M, N, K, seed=M + N + K)
    bits, info = run_gemm(A, B, M, N, K, "bf16", out, "bn", return_plan_info=True)
    assert info["tile_m"] == (128 if tile == "generic128" else 256)
    C, _ = oracle_mod.gemm_ab(A, B)
    _exact(oracle_mod, bits, out, C)


@pytest.mark.parametrize("tile", ["tile256", "generic256", "generic128"])
def test_bn_random_within_bound(oracle_mod, monkeypatch, tile):
    M, N, K = 520, 784, 1504
    set_tile(monkeypatch, tile)
    say("case bn random", tile, M, N, K)
    inp = W.make_inputs(W.WORKLOADS["bf16_4096_bn"], M=M, N=N, K=K, seed=41)
    assert inp.B.shape == (K, N)
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", "bn")
    C, S = oracle_mod.gemm_ab(inp.A, inp.B)
    r = assert_within_bound(decode(bits), C, S, "bf16", "bn random " + tile)
    say("  worst err/bound", r)


def test_bn_with_epilogue(oracle_mod, monkeypatch):
    M, N, K = 300, 272, 1056
    set_tile(monkeypatch, None)
    say("case bn epilogue", M, N, K)
    inp = W.make_inputs(W.WORKLOADS["bf16_4096_bn"], M=M, N=N, K=K, seed=43)
    rng = np.random.default_rng(44)
    e = dict(scale_a=rng.uniform(0.05, 0.1, M), scale_b=rng.uniform(0.5, 2.0, N), bias=rng.normal(0, 1, N),
             kind="bias_gelu")
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", "bn", epi=e)
    acc, S = oracle_mod.gemm_ab(inp.A, inp.B)
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e["bias"], e["kind"])
    scale = np.abs(e["scale_a"][:, None] * e["scale_b"][None, :])
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"])[None, :], "bf16", "bias_gelu", "bn epilogue")
    say("  worst err/bound", r)


def test_bn_full_size_sampled(oracle_mod, monkeypatch):
    set_tile(monkeypatch, None)
    w = W.WORKLOADS["bf16_4096_bn"]
    say("case bn full-size", w.name)
    inp = W.make_inputs(w)
    bits = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    C, S = oracle_mod.gemm_ab_entries(inp.A, inp.B, rows, cols)
    r = assert_within_bound(decode(bits[rows, cols]), C, S, "bf16", w.name)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))


# ------------------------------------------------------------------ fp8 e4m3 (8-bit transpose read)

@pytest.mark.parametrize("M,N,K", [(300, 272, 1088), (256, 512, 1024), (1, 16, 64), (77, 48, 192)])
def test_bn_fp8_bit_exact(oracle_mod, monkeypatch, M, N, K):
    # integer values in [-4, 4] are exact in e4m3; power-of-two scales keep
    # the sums and the scaled result exact, so the bf16 output is the single
    # RNE of an exact value on both sides
    set_tile(monkeypatch, None)
    say("case bn fp8 exact", M, N, K)
    inp = W.int_inputs(M, N, K, "e4m3", seed=M + 3 * N + K)
    B_kn = np.ascontiguousarray(inp.B.T)
    bits, info = run_gemm(inp.A, B_kn, M, N, K, "e4m3", "bf16", "bn", scale=(0.5, 0.25), return_plan_info=True)
    assert info["tile_m"] == 256
    C, _ = oracle_mod.gemm_ab(inp.A, B_kn, dtype="e4m3", sigma=oracle_mod.sigma_of(0.5, 0.25))
    _exact(oracle_mod, bits, "bf16", C)


@pytest.mark.parametrize("M,N,K", [(520, 784, 1536), (4096, 4096, 4096)])
def test_bn_fp8_random_within_bound(oracle_mod, monkeypatch, M, N, K):
    set_tile(monkeypatch, None)
    say("case bn fp8 random", M, N, K)
    inp = W.make_inputs(W.WORKLOADS["e4m3_8192"], M=M, N=N, K=K, seed=53)
    B_kn = np.ascontiguousarray(inp.B.T)
    bits = run_gemm(inp.A, B_kn, M, N, K, "e4m3", "bf16", "bn", scale=(inp.scale_a, inp.scale_b))
    sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
    if M * N <= 1 << 20:
        C, S = oracle_mod.gemm_ab(inp.A, B_kn, dtype="e4m3", sigma=sigma)
        got = decode(bits)
    else:
        rows, cols = block_entries(M, N, seed=54)
        C, S = oracle_mod.gemm_ab_entries(inp.A, B_kn, rows, cols, dtype="e4m3", sigma=sigma)
        got = decode(bits[rows, cols])
        assert np.all(np.isfinite(decode(bits)))
    r = assert_within_bound(got, C, S, "e4m3", "bn fp8 random %dx%dx%d" % (M, N, K))
    say("  worst err/bound", r)


# ------------------------------------------------------------------ int8 (8-bit transpose read, int32 sums)

@pytest.mark.parametrize("M,N,K", [(300, 272, 1088), (256, 512, 1024), (1, 16, 64), (77, 48, 192)])
def test_bn_int8_bit_exact(oracle_mod, monkeypatch, M, N, K):
    # full-range int8 with sums of |a b| below 2^24: the bf16 output is the
    # single RNE of the exact int32 sum, dequantised by per-row / per-column
    # powers of two; B is handed over K x N, the oracle takes the N x K copy
    set_tile(monkeypatch, None)
    say("case bn int8 exact", M, N, K)
    inp = W.int_inputs(M, N, K, "i8", seed=M + 5 * N + K, lo=-128, hi=127)
    B_kn = np.ascontiguousarray(inp.B.T)
    rng = np.random.default_rng(M + N)
    e = dict(scale_a=2.0 ** rng.integers(-3, 1, M), scale_b=2.0 ** rng.integers(-3, 1, N), kind="none")
    bits, info = run_gemm(inp.A, B_kn, M, N, K, "i8", "bf16", "bn", epi=e, return_plan_info=True)
    assert info["tile_m"] == 256 and info["kernel"] == 0
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, "i8")
    assert S.max() < 2.0 ** 24
    want = oracle_mod.round_bf16(oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], None, "none"))
    bad = np.argwhere(bits != want)
    assert bad.size == 0, "%d mismatches, first %s" % (len(bad), bad[:3].tolist())


def test_bn_int8_quantised_full_size_sampled(oracle_mod, monkeypatch):
    set_tile(monkeypatch, None)
    M = N = K = 4096
    say("case bn int8 quantised", M, N, K)
    inp = W.make_inputs(W.WORKLOADS["i8_8192"], M=M, N=N, K=K, seed=61)
    B_kn = np.ascontiguousarray(inp.B.T)
    e = dict(scale_a=inp.sa_rows.astype(np.float64), scale_b=inp.sb_cols.astype(np.float64), kind="none")
    bits = run_gemm(inp.A, B_kn, M, N, K, "i8", "bf16", "bn", epi=e)
    rows, cols = block_entries(M, N, seed=62)
    acc, S = oracle_mod.gemm_bt_int_entries(inp.A, inp.B, K, rows, cols, "i8")
    want = oracle_mod.epilogue_entries(acc, e["scale_a"][rows], e["scale_b"][cols], None, "none")
    scale = np.abs(e["scale_a"][rows] * e["scale_b"][cols])
    r = assert_epilogue_within_bound(decode(bits[rows, cols]), want, S * scale, np.abs(acc) * scale, 0.0, "i8",
                                     "none", "bn int8 4096^3")
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))
