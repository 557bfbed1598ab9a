"""Parity of C = A * B^T with A stored K x M (GEMM_LAYOUT_AT, B N x K;
GEMM_LAYOUT_AT_BN, B K x N), both read through the LDS transpose load, with
the oracle's gemm_at.

* Integer-valued bf16 inputs (exact sums): bit-exact for both outputs, with
  M and N tails inside a 256 x 256 tile, a half-filled last K step
  (K % 64 == 32) and the smallest shapes.
* N(0,1) inputs: within the GEMM bound; the 4096^3 workloads on sampled
  entries; a fused epilogue.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_epilogue_within_bound, assert_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu

LAYOUTS = ["at", "at_bn"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


def int_at(M, N, K, layout, seed):
    """Integer-valued bf16 A stored K x M and B (N x K, or K x N for at_bn)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-4, 5, (K, M)).astype(np.float32)
    b = rng.integers(-4, 5, (K, N) if layout == "at_bn" else (N, K)).astype(np.float32)
    return W.to_bf16_bits(a), W.to_bf16_bits(b)


def _exact(oracle_mod, bits, out, C):
    if out == "f32":
        want = C.astype(np.float32).view(np.uint32)
    else:
        want = oracle_mod.round_bf16(C)
    bad = bits != want
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])], C[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(296, 272, 1056), (256, 512, 1024), (8, 16, 32), (520, 48, 96)])
def test_at_bit_exact(oracle_mod, layout, out, M, N, K):
    say("case at exact", layout, out, M, N, K)
    A, B = int_at(M, N, K, layout, seed=M + N + K)
    bits, info = run_gemm(A, B, M, N, K, "bf16", out, layout, return_plan_info=True)
    assert info["tile_m"] == 256 and info["threads"] == 512
    C, _ = oracle_mod.gemm_at(A, B, b_kn=layout == "at_bn")
    _exact(oracle_mod, bits, out, C)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_at_random_within_bound(oracle_mod, layout):
    M, N, K = 520, 784, 1504
    say("case at random", layout, M, N, K)
    inp = W.make_inputs(W.WORKLOADS["bf16_4096_" + layout], M=M, N=N, K=K, seed=47)
    assert inp.A.shape == (K, M)
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", layout)
    C, S = oracle_mod.gemm_at(inp.A, inp.B, b_kn=layout == "at_bn")
    r = assert_within_bound(decode(bits), C, S, "bf16", "at random " + layout)
    say("  worst err/bound", r)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_at_with_epilogue(oracle_mod, layout):
    M, N, K = 296, 272, 1056
    say("case at epilogue", layout, M, N, K)
    inp = W.make_inputs(W.WORKLOADS["bf16_4096_" + layout], M=M, N=N, K=K, seed=49)
    rng = np.random.default_rng(50)
    e = dict(scale_a=rng.uniform(0.05, 0.1, M), scale_b=rng.uniform(0.5, 2.0, N), bias=rng.normal(0, 1, N),
             kind="bias_silu")
    bits = run_gemm(inp.A, inp.B, M, N, K, "bf16", "bf16", layout, epi=e)
    acc, S = oracle_mod.gemm_at(inp.A, inp.B, b_kn=layout == "at_bn")
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e["bias"], e["kind"])
    scale = np.abs(e["scale_a"][:, None] * e["scale_b"][None, :])
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"])[None, :], "bf16", "bias_silu", "at epilogue")
    say("  worst err/bound", r)


@pytest.mark.parametrize("name", ["bf16_4096_at", "bf16_4096_at_bn"])
def test_at_full_size_sampled(oracle_mod, name):
    w = W.WORKLOADS[name]
    say("case at full-size", w.name)
    inp = W.make_inputs(w)
    bits = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    C, S = oracle_mod.gemm_at_entries(inp.A, inp.B, rows, cols, b_kn=w.layout == "at_bn")
    r = assert_within_bound(decode(bits[rows, cols]), C, S, "bf16", w.name)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))


# ------------------------------------------------------------------ 8-bit A stored K x M (8-bit transpose reads)

EIGHT_BIT_SHAPES = [(304, 272, 1088), (256, 512, 1024), (16, 16, 64), (528, 48, 192)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", EIGHT_BIT_SHAPES)
def test_at_fp8_bit_exact(oracle_mod, layout, M, N, K):
    # e4m3 integers in [-4, 4] and power-of-two scales: exact sums, one RNE
    say("case at fp8 exact", layout, M, N, K)
    inp = W.int_inputs(M, N, K, "e4m3", seed=M + 7 * N + K)
    A_km = np.ascontiguousarray(inp.A.T)
    B = np.ascontiguousarray(inp.B.T) if layout == "at_bn" else inp.B
    bits, info = run_gemm(A_km, B, M, N, K, "e4m3", "bf16", layout, scale=(0.5, 0.25), return_plan_info=True)
    assert info["tile_m"] == 256
    C, _ = oracle_mod.gemm_at(A_km, B, dtype="e4m3", sigma=oracle_mod.sigma_of(0.5, 0.25), want_s=False,
                              b_kn=layout == "at_bn")
    _exact(oracle_mod, bits, "bf16", C)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", EIGHT_BIT_SHAPES)
def test_at_int8_bit_exact(oracle_mod, layout, M, N, K):
    # full-range int8 with sums of |a b| below 2^24: exact int32 sums, one RNE
    say("case at int8 exact", layout, M, N, K)
    inp = W.int_inputs(M, N, K, "i8", seed=M + 11 * N + K, lo=-128, hi=127)
    A_km = np.ascontiguousarray(inp.A.T)
    B = np.ascontiguousarray(inp.B.T) if layout == "at_bn" else inp.B
    bits = run_gemm(A_km, B, M, N, K, "i8", "bf16", layout)
    acc, S = oracle_mod.gemm_bt_int(inp.A, inp.B, K, "i8")
    assert S.max() < 2.0 ** 24
    _exact(oracle_mod, bits, "bf16", acc)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_at_fp8_random_4096_sampled(oracle_mod, layout):
    M = N = K = 4096
    say("case at fp8 random", layout, M, N, K)
    inp = W.make_inputs(W.WORKLOADS["e4m3_8192"], M=M, N=N, K=K, seed=71)
    A_km = np.ascontiguousarray(inp.A.T)
    B = np.ascontiguousarray(inp.B.T) if layout == "at_bn" else inp.B
    bits = run_gemm(A_km, B, M, N, K, "e4m3", "bf16", layout, scale=(inp.scale_a, inp.scale_b))
    rows, cols = block_entries(M, N, seed=72)
    sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
    C, S = oracle_mod.gemm_at_entries(A_km, B, rows, cols, dtype="e4m3", sigma=sigma, b_kn=layout == "at_bn")
    r = assert_within_bound(decode(bits[rows, cols]), C, S, "e4m3", "at fp8 %s 4096^3" % layout)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))
