"""Parity of the MX block-scaled GEMM (gemm_preshuffle_bscale + gemm_run_mx)
with the oracle.

* The block-scale image is a byte permutation: byte-exact against
  oracle.layout.bscale_image, with ragged rows and K.
* Small MX inputs whose products and sums are exact in fp32 (e4m3 integers or
  any e2m1 code, scales 2^-2 .. 2^2): bit-exact C, plain and pre-shuffled B,
  a half-filled last K step, and with a fused epilogue.
* Random MX inputs: within the GEMM bound; the full-size workloads sampled.
"""
import numpy as np
import pytest
import torch

import tiled_gemm_amd as tg
import workloads as W
import gpu_util
from gpu_util import assert_epilogue_within_bound, assert_within_bound, decode, run_gemm, block_entries
from oracle import layout as OL

pytestmark = pytest.mark.gpu

FMTS = ["mxfp8", "mxfp4"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("R,K", [(200, 1088), (64, 128), (513, 4096)])
def test_bscale_image_byte_exact(monkeypatch, R, K):
    # form 0: the 16x16x128 kernels' image (the skinny MX kernels, and the
    # 4-wave tile kernel)
    say("case bscale image", R, K)
    gpu_util.force("pipe4")
    rng = np.random.default_rng(R + K)
    S = rng.integers(0, 255, (R, K // 32)).astype(np.uint8)
    with gpu_util.plan(R, 64, K, tg.GEMM_MXFP8_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert p.info()["scale_form"] == 0
        n = p.bscale_image_bytes(0)
        src = torch.from_numpy(S).cuda()
        img = torch.full((n,), 0xEE, dtype=torch.uint8, device="cuda")
        p.preshuffle_bscale(0, src.data_ptr(), img.data_ptr())
        torch.cuda.synchronize()
        got = img.cpu().numpy()
    want = OL.bscale_image(S, K)
    assert got.size == want.size
    assert np.array_equal(got, want)


@pytest.mark.parametrize("R,K", [(200, 1152), (513, 4096)])
def test_bscale_image_form1_byte_exact(R, K):
    # MX on 256 x 256 tiles runs the 32x32x64 kernel, whose plan writes form 1.
    say("case bscale image form 1", R, K)
    rng = np.random.default_rng(R * K)
    S = rng.integers(0, 255, (R, K // 32)).astype(np.uint8)
    with tg.Plan(R, 512, K, tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED) as p:
        assert p.info()["scale_form"] == 1 and p.info()["tile_m"] == 256
        n = p.bscale_image_bytes(0)
        src = torch.from_numpy(S).cuda()
        img = torch.full((n,), 0xEE, dtype=torch.uint8, device="cuda")
        p.preshuffle_bscale(0, src.data_ptr(), img.data_ptr())
        torch.cuda.synchronize()
        got = img.cpu().numpy()
    want = OL.bscale_image_32(S, K)
    assert got.size == want.size
    assert np.array_equal(got, want)


def _k_for(fmt, ragged):
    # ragged: K bytes an odd multiple of 64, so the last 128-byte step is half full
    if fmt == "mxfp8":
        return 1088 if ragged else 1024
    return 1152 if ragged else 1024


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("ragged", [False, True])
def test_mx_bit_exact(oracle_mod, fmt, layout, ragged):
    M, N, K = 300, 272, _k_for(fmt, ragged)
    say("case mx exact", fmt, layout, M, N, K)
    inp = W.mx_int_inputs(M, N, K, fmt, seed=K + len(layout))
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, sa_blocks=inp.sa_blocks,
                          sb_blocks=inp.sb_blocks, return_plan_info=True)
    assert info["elem_bits"] == (8 if fmt == "mxfp8" else 4)
    C, S = oracle_mod.gemm_bt_mx(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, K, fmt)
    assert S.max() < 2.0 ** 18          # every partial sum exact in fp32 (granularity >= 2^-6)
    want = oracle_mod.round_bf16(C)
    bad = bits != want
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])], C[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_with_epilogue_bit_exact(oracle_mod, fmt):
    M, N, K = 300, 272, _k_for(fmt, True)
    say("case mx epilogue exact", fmt, M, N, K)
    inp = W.mx_int_inputs(M, N, K, fmt, seed=99)
    rng = np.random.default_rng(5)
    e = dict(scale_a=2.0 ** rng.integers(-2, 3, M), scale_b=2.0 ** rng.integers(-2, 3, N),
             bias=rng.integers(-8, 9, N).astype(np.float64), kind="bias_relu")
    bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", "bt_preshuffled", sa_blocks=inp.sa_blocks,
                    sb_blocks=inp.sb_blocks, epi=e)
    C, _ = oracle_mod.gemm_bt_mx(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, K, fmt)
    want = oracle_mod.round_bf16(oracle_mod.epilogue(C, e["scale_a"], e["scale_b"], e["bias"], e["kind"]))
    assert np.array_equal(bits, want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
def test_mx_random_within_bound(oracle_mod, fmt, layout):
    M, N, K = 520, 784, 1536
    say("case mx random", fmt, layout, M, N, K)
    inp = W.make_inputs(W.WORKLOADS[fmt + "_8192"], M=M, N=N, K=K, seed=31)
    bits = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", layout, sa_blocks=inp.sa_blocks, sb_blocks=inp.sb_blocks)
    C, S = oracle_mod.gemm_bt_mx(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, K, fmt)
    r = assert_within_bound(decode(bits), C, S, fmt, "mx random %s %s" % (fmt, layout))
    say("  worst err/bound", r)


# Decode shapes (M <= 64) with B pre-shuffled run on the skinny kernel: the
# waves split K in whole scale groups, the scale words ride with each stage.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 17, 32, 33, 64])
@pytest.mark.parametrize("N,ragged", [(544, False), (528, True)])
def test_mx_skinny_bit_exact(oracle_mod, fmt, M, N, ragged):
    K = _k_for(fmt, ragged)
    say("case mx skinny exact", fmt, M, N, K)
    inp = W.mx_int_inputs(M, N, K, fmt, seed=M + N + K)
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", "bt_preshuffled", sa_blocks=inp.sa_blocks,
                          sb_blocks=inp.sb_blocks, return_plan_info=True)
    assert info["kernel"] == 1
    C, S = oracle_mod.gemm_bt_mx(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, K, fmt)
    assert S.max() < 2.0 ** 18
    want = oracle_mod.round_bf16(C)
    bad = bits != want
    assert not bad.any(), "%d mismatches, first at %s: got %r want %r" % (
        int(bad.sum()), np.argwhere(bad)[0], decode(bits)[tuple(np.argwhere(bad)[0])], C[tuple(np.argwhere(bad)[0])])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [8, 48])
def test_mx_skinny_random_within_bound(oracle_mod, fmt, M):
    N, K = 784, 4096
    say("case mx skinny random", fmt, M, N, K)
    inp = W.make_inputs(W.WORKLOADS[fmt + "_8192"], M=M, N=N, K=K, seed=57)
    e = dict(scale_a=np.full(M, 0.5), scale_b=np.linspace(0.5, 2.0, N), bias=np.linspace(-1.0, 1.0, N),
             kind="bias_silu")
    bits, info = run_gemm(inp.A, inp.B, M, N, K, fmt, "bf16", "bt_preshuffled", sa_blocks=inp.sa_blocks,
                          sb_blocks=inp.sb_blocks, epi=e, return_plan_info=True)
    assert info["kernel"] == 1
    acc, S = oracle_mod.gemm_bt_mx(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, K, fmt)
    want = oracle_mod.epilogue(acc, e["scale_a"], e["scale_b"], e["bias"], e["kind"])
    scale = np.abs(e["scale_a"][:, None] * e["scale_b"][None, :])
    r = assert_epilogue_within_bound(decode(bits), want, S * scale, np.abs(acc) * scale,
                                     np.abs(e["bias"])[None, :], fmt, e["kind"], "mx skinny " + fmt)
    say("  worst err/bound", r)


def test_mx_plain_decode_stays_tiled():
    with tg.Plan(32, 8192, 8192, tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert p.info()["kernel"] == 0


@pytest.mark.parametrize("name,kind", [("mxfp8_8192", "none"), ("mxfp4_8192", "none"), ("mxfp4_8192", "bias_gelu"),
                                       ("mxfp4_32x8192x8192", "none")])
def test_mx_full_size_sampled(oracle_mod, name, kind):
    w = W.WORKLOADS[name]
    say("case mx full-size", name, kind)
    inp = W.make_inputs(w)
    e = None
    if kind != "none":
        rng = np.random.default_rng(w.seed + 1)
        e = dict(scale_a=rng.uniform(0.01, 0.05, w.M), scale_b=rng.uniform(0.5, 2.0, w.N),
                 bias=rng.normal(0.0, 1.0, w.N), kind=kind)
    bits = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout, sa_blocks=inp.sa_blocks,
                    sb_blocks=inp.sb_blocks, epi=e)
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    acc, S = oracle_mod.gemm_bt_mx_entries(inp.A, inp.sa_blocks, inp.B, inp.sb_blocks, w.K, rows, cols, w.dtype)
    got = decode(bits[rows, cols])
    if e is None:
        r = assert_within_bound(got, acc, S, w.dtype, name)
    else:
        want = oracle_mod.epilogue_entries(acc, e["scale_a"][rows], e["scale_b"][cols], e["bias"][cols], kind)
        scale = np.abs(e["scale_a"][rows] * e["scale_b"][cols])
        r = assert_epilogue_within_bound(got, want, S * scale, np.abs(acc) * scale, np.abs(e["bias"][cols]),
                                         w.dtype, kind, name)
    say("  worst err/bound", r)
    assert np.all(np.isfinite(decode(bits)))
