"""Parity of the fused epilogue (gemm_run_ex) with the oracle's epilogue.

* Integer inputs, power-of-two scales and integer bias: every intermediate
  value is exact in fp32, so "none", "bias" and "bias_relu" must match the
  oracle bit for bit on every kernel path, for each scale granularity
  (per row / per column / one value / absent).
* SiLU and GELU on random inputs: the GEMM bound carried through the
  activation (gpu_util.assert_epilogue_within_bound).
* The full-size workloads with an epilogue, on sampled entries.
"""
import numpy as np
import pytest
import torch

import workloads as W
import gpu_util
from gpu_util import assert_epilogue_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu

# (tile env, layout, M): "256x256" the planner's 256 x 256 kernel (bf16 with
# B stored N x K: both operands through LDS; fp8: pipelined 8-wave),
# "256x256p" pipelined 8-wave with B in registers, "256x256q" pipelined
# 4-wave, "256x256g" generic, "128x128" generic, None with M <= 64 skinny.
PATHS = [("tile256", "bt", None), ("pipe", "bt", None), ("pipe4", "bt_preshuffled", None), ("generic256", "bt", None),
         ("generic128", "bt_preshuffled", None), (None, "bt", 33), (None, "bt_preshuffled", 33)]
DTYPES = [("bf16", "f32"), ("bf16", "bf16"), ("e4m3", "bf16")]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


def set_path(monkeypatch, kernel):
    gpu_util.force(kernel)


def epi_case(name, M, N, rng):
    """Scale vectors / scalars / None and integer bias for one exactness case."""
    p2 = lambda n: (2.0 ** rng.integers(-2, 3, n)) * rng.choice([-1.0, 1.0], n)
    cases = {
        "rowcol_none": dict(scale_a=p2(M), scale_b=p2(N), kind="none"),
        "scalar_bias": dict(scale_a=0.25, scale_b=-2.0, kind="bias"),
        "row_relu": dict(scale_a=p2(M), kind="bias_relu"),
        "col_relu": dict(scale_b=p2(N), kind="bias_relu"),
        "rowcol_bias": dict(scale_a=p2(M), scale_b=p2(N), kind="bias"),
    }
    e = dict(cases[name])
    if e["kind"] != "none":
        e["bias"] = rng.integers(-8, 9, N).astype(np.float64)
    return e


def expected(oracle_mod, acc, e):
    return oracle_mod.epilogue(acc, e.get("scale_a"), e.get("scale_b"), e.get("bias"), e["kind"])


@pytest.mark.parametrize("tile,layout,m_skinny", PATHS)
@pytest.mark.parametrize("dtype,out", DTYPES)
@pytest.mark.parametrize("case", ["rowcol_none", "scalar_bias", "row_relu", "col_relu", "rowcol_bias"])
def test_epilogue_bit_exact(oracle_mod, monkeypatch, tile, layout, m_skinny, dtype, out, case):
    M = m_skinny or 300
    N, K = 272, (1056 if dtype == "bf16" else 1088)     # K*e an odd multiple of 64: half-filled last step
    set_path(monkeypatch, tile)
    say("case epilogue exact", tile, layout, dtype, out, case, M, N, K)
    rng = np.random.default_rng(M * 31 + len(case))
    inp = W.int_inputs(M, N, K, dtype, seed=M + N + K + len(case))
    e = epi_case(case, M, N, rng)
    bits, info = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, epi=e, return_plan_info=True)
    if m_skinny:
        assert info["kernel"] == 1
    acc, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype)
    want = expected(oracle_mod, acc, e)
    if out == "f32":
        ref = want.astype(np.float32).view(np.uint32)
        assert np.array_equal(want.astype(np.float32).astype(np.float64), want)   # exact in fp32
    else:
        ref = oracle_mod.round_bf16(want)
    bad = bits != ref
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])],
        want[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("tile,layout,m_skinny", PATHS)
@pytest.mark.parametrize("dtype,out", DTYPES)
@pytest.mark.parametrize("kind", ["bias_silu", "bias_gelu"])
def test_epilogue_smooth_within_bound(oracle_mod, monkeypatch, tile, layout, m_skinny, dtype, out, kind):
    M = m_skinny or 520
    N, K = 784, 1472
    set_path(monkeypatch, tile)
    say("case epilogue random", tile, layout, dtype, out, kind, M, N, K)
    w = W.WORKLOADS["e4m3_8192" if dtype == "e4m3" else "bf16_4096"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=777)
    rng = np.random.default_rng(778)
    # pre-activation values mostly in |z| < 6, where SiLU and GELU bend
    sa = rng.uniform(0.02, 0.1, M) * inp.scale_a
    sb = rng.uniform(0.5, 2.0, N) * inp.scale_b
    e = dict(scale_a=sa, scale_b=sb, bias=rng.normal(0.0, 1.0, N), kind=kind)
    bits = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, epi=e)
    acc, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype)
    want = expected(oracle_mod, acc, e)
    scale = np.abs(sa[:, None] * sb[None, :])
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"])[None, :], dtype, kind, "%s %s %s" % (tile, dtype, kind))
    say("  worst err/bound", r)


@pytest.mark.parametrize("name,kind", [("bf16_8192_preshuffled", "bias_gelu"), ("e4m3_8192", "bias_silu"),
                                       ("bf16_skinny_32x8192x8192", "bias_relu"), ("bf16_4096", "bias")])
def test_epilogue_full_size_sampled(oracle_mod, monkeypatch, name, kind):
    set_path(monkeypatch, None)
    w = W.WORKLOADS[name]
    say("case epilogue full-size", name, kind)
    inp = W.make_inputs(w)
    rng = np.random.default_rng(w.seed + 1)
    sa = rng.uniform(0.01, 0.05, w.M) * inp.scale_a
    sb = rng.uniform(0.5, 2.0, w.N) * inp.scale_b
    e = dict(scale_a=sa, scale_b=sb, bias=rng.normal(0.0, 1.0, w.N), kind=kind)
    bits = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout, epi=e)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    acc, S = oracle_mod.gemm_bt_entries(inp.A, inp.B, rows, cols, dtype=w.dtype)
    want = oracle_mod.epilogue_entries(acc, sa[rows], sb[cols], e["bias"][cols], kind)
    scale = np.abs(sa[rows] * sb[cols])
    r = assert_epilogue_within_bound(decode(bits[rows, cols]), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"][cols]), w.dtype, kind, name)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))


def test_epilogue_none_equals_gemm_run(monkeypatch):
    """gemm_run(scale) is gemm_run_ex with the two scalars and no activation."""
    set_path(monkeypatch, None)
    M, N, K = 300, 272, 192
    inp = W.int_inputs(M, N, K, "e4m3", seed=5)
    a = run_gemm(inp.A, inp.B, M, N, K, "e4m3", "bf16", "bt", scale=(0.5, 0.25))
    b = run_gemm(inp.A, inp.B, M, N, K, "e4m3", "bf16", "bt", epi=dict(scale_a=0.5, scale_b=0.25, kind="none"))
    assert np.array_equal(a, b)
