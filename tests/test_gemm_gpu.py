"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact where the arithmetic is exact (integer-valued inputs whose partial
sums fit fp32), within the stated bound otherwise.  Shapes span several
tiles with ragged M, N and K tails; the full-size workloads run in the
launch configuration the benchmark times and are checked on sampled entries.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import tiled_gemm_amd as tg
import workloads as W
from gpu_util import assert_within_bound, decode, run_gemm, block_entries

pytestmark = pytest.mark.gpu

# (dtype, out, layout, kernel) -- kernel: a gemm_kernel_choice name (None = the
# planner's own choice): "tile256" the planner's 256 x 256 kernel (bf16 with B
# stored N x K: both operands through LDS; otherwise the software-pipelined
# kernel), "pipe" the software-pipelined kernel with B in registers,
# "generic128" / "generic256" the generic tiled kernel, "pipe4" the 4-wave
# pipelined kernel.
PATHS = [
    ("bf16", "f32", "bt", "generic128"), ("bf16", "f32", "bt", "tile256"), ("bf16", "f32", "bt", "generic256"),
    ("bf16", "bf16", "bt", "generic128"), ("bf16", "bf16", "bt", "tile256"), ("bf16", "bf16", "bt", "generic256"),
    ("bf16", "bf16", "bt_preshuffled", "generic128"), ("bf16", "bf16", "bt_preshuffled", "tile256"),
    ("bf16", "bf16", "bt_preshuffled", "generic256"), ("bf16", "f32", "bt_preshuffled", "tile256"),
    ("e4m3", "bf16", "bt", "generic128"), ("e4m3", "bf16", "bt", "tile256"), ("e4m3", "bf16", "bt", "generic256"),
    ("e4m3", "bf16", "bt_preshuffled", "generic128"), ("e4m3", "bf16", "bt_preshuffled", "tile256"),
    ("e4m3", "bf16", "bt_preshuffled", "generic256"),
    ("bf16", "f32", "bt", "pipe4"), ("bf16", "bf16", "bt", "pipe4"),
    ("bf16", "bf16", "bt_preshuffled", "pipe4"), ("bf16", "f32", "bt_preshuffled", "pipe4"),
    ("e4m3", "bf16", "bt", "pipe4"), ("e4m3", "bf16", "bt_preshuffled", "pipe4"),
    ("bf16", "f32", "bt", "pipe"), ("bf16", "bf16", "bt", "pipe"),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.fixture
def tile_env(plan_opts):
    """Kernel choice for the plans run_gemm creates (None: the planner's)."""
    return lambda kernel: plan_opts(kernel=kernel)


def exact_check(oracle_mod, inp, M, N, K, dtype, out, layout, scale=(1.0, 1.0)):
    C_bits = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, scale=scale)
    sigma = oracle_mod.sigma_of(*scale)
    C_ref, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype, sigma=sigma, want_s=False)
    if out == "f32":
        want = C_ref.astype(np.float32)
        assert np.array_equal(want.astype(np.float64), C_ref), "reference not exact in fp32"
        got = C_bits.view(np.float32)
        bad = np.argwhere(got != want)
        assert bad.size == 0, "first mismatches %s: got %s want %s" % (
            bad[:3].tolist(), got[tuple(bad[0])], want[tuple(bad[0])])
    else:
        want = oracle_mod.round_bf16(C_ref)
        bad = np.argwhere(C_bits != want)
        assert bad.size == 0, "first mismatches %s: got %s want %s (ref %r)" % (
            bad[:3].tolist(), hex(C_bits[tuple(bad[0])]), hex(want[tuple(bad[0])]), C_ref[tuple(bad[0])])


# ------------------------------------------------------------------ config 1

def test_bf16_int_256_bit_exact(oracle_mod):
    w = W.WORKLOADS["bf16_int_256"]
    say("case bf16_int_256", w)
    inp = W.make_inputs(w)
    exact_check(oracle_mod, inp, w.M, w.N, w.K, "bf16", "f32", "bt")


# ------------------------------------------------------------------ integer-exact, every path

@pytest.mark.parametrize("dtype,out,layout,tile", PATHS)
@pytest.mark.parametrize("shape", ["small", "ragged"])
def test_integer_exact_every_path(oracle_mod, tile_env, dtype, out, layout, tile, shape):
    # "ragged": M and N not multiples of the tile, and K*elem_bytes an odd
    # multiple of 64 so the last 128-byte K step is half full.
    if shape == "small":
        M, N, K = 300, 272, 192
    else:
        M, N, K = 513, 528, (1056 if dtype == "bf16" else 1088)
    tile_env(tile)
    say("case int-exact", dtype, out, layout, tile, M, N, K)
    inp = W.int_inputs(M, N, K, dtype, seed=M * 7 + N + K)
    scale = (0.5, 0.25) if dtype == "e4m3" else (1.0, 1.0)
    exact_check(oracle_mod, inp, M, N, K, dtype, out, layout, scale)


@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("e4m3", "bf16")])
@pytest.mark.parametrize("M", [1, 17, 32, 33, 64])
@pytest.mark.parametrize("N,kpad", [(544, 0), (528, 64)])
def test_integer_exact_skinny(oracle_mod, tile_env, dtype, out, M, layout, N, kpad):
    # kpad = 64: K * elem_bytes is an odd multiple of 64, so the last 128-byte
    # K step is half full; N = 528 leaves the last workgroup one 16-column block.
    tile_env(None)
    K = (1024 + kpad) // (2 if dtype == "bf16" else 1)
    say("case skinny int-exact", dtype, out, layout, M, N, K)
    inp = W.int_inputs(M, N, K, dtype, seed=M + N + 99)
    with tg.Plan(M, N, K, gpu_dtype(dtype, out), tg.LAYOUTS[layout]) as p:
        assert p.info()["kernel"] == 1
    scale = (2.0, 0.125) if dtype == "e4m3" else (1.0, 1.0)
    exact_check(oracle_mod, inp, M, N, K, dtype, out, layout, scale)


@pytest.mark.parametrize("layout", ["bt", "bt_preshuffled"])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("e4m3", "bf16")])
@pytest.mark.parametrize("M", [1, 32, 64])
def test_random_skinny(oracle_mod, tile_env, dtype, out, M, layout):
    N, K = 784, 2080 if dtype == "bf16" else 4160
    tile_env(None)
    say("case skinny random", dtype, out, layout, M, N, K)
    w = W.WORKLOADS["e4m3_8192" if dtype == "e4m3" else "bf16_skinny_32x8192x8192"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=777 + M)
    C_bits, info = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, scale=(inp.scale_a, inp.scale_b),
                            return_plan_info=True)
    assert info["kernel"] == 1
    sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
    C_ref, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype, sigma=sigma)
    r = assert_within_bound(decode(C_bits), C_ref, S, dtype, "skinny random %s %s M=%d" % (dtype, layout, M))
    say("  worst err/bound", r)


def gpu_dtype(dtype, out):
    return {("bf16", "f32"): tg.GEMM_BF16_OUT_F32, ("bf16", "bf16"): tg.GEMM_BF16_OUT_BF16,
            ("e4m3", "bf16"): tg.GEMM_E4M3_OUT_BF16}[(dtype, out)]


# ------------------------------------------------------------------ random values, full oracle

@pytest.mark.parametrize("dtype,out,layout,tile", PATHS + [("bf16", "bf16", "bt", None), ("e4m3", "bf16", "bt", None)])
def test_random_within_bound(oracle_mod, tile_env, dtype, out, layout, tile):
    M, N, K = 520, 784, 1472
    tile_env(tile)
    say("case random", dtype, out, layout, tile, M, N, K)
    w = W.WORKLOADS["e4m3_8192" if dtype == "e4m3" else "bf16_4096"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=4242)
    C_bits = run_gemm(inp.A, inp.B, M, N, K, dtype, out, layout, scale=(inp.scale_a, inp.scale_b))
    sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
    C_ref, S = oracle_mod.gemm_bt(inp.A, inp.B, dtype=dtype, sigma=sigma)
    r = assert_within_bound(decode(C_bits), C_ref, S, dtype, "random %s %s %s" % (dtype, layout, tile))
    say("  worst err/bound", r)


# ------------------------------------------------------------------ full-size workloads

# Workloads whose whole C the oracle computes within seconds on the host: the
# 4096^3 GEMM (1.4e11 multiply-adds) and the decode shapes.  The 8192^3 ones
# are checked on one entry of every 16 x 16 block of C plus the border rows
# and columns (gpu_util.block_entries).
FULL_C = ("bf16_4096", "bf16_skinny_32x8192x8192", "bf16_skinny_32x8192x8192_preshuffled")
_full_ref = {}


def _oracle_full(oracle_mod, name, inp):
    if name not in _full_ref:
        w = W.WORKLOADS[name]
        t0 = time.perf_counter()
        sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
        _full_ref[name] = oracle_mod.gemm_bt(inp.A, inp.B, dtype=w.dtype, sigma=sigma)
        say("  oracle: whole C of %s in %.1f s on %d threads" % (name, time.perf_counter() - t0,
                                                                 oracle_mod.threads()))
    return _full_ref[name]


@pytest.mark.parametrize("name,tile", [("bf16_4096", None), ("bf16_4096", "pipe"), ("bf16_4096", "pipe4"),
                                       ("bf16_8192_preshuffled", None), ("bf16_8192_preshuffled", "pipe4"),
                                       ("bf16_skinny_32x8192x8192", None),
                                       ("bf16_skinny_32x8192x8192_preshuffled", None), ("e4m3_8192", None),
                                       ("e4m3_8192", "pipe4"), ("e4m3_8192_preshuffled", None)])
def test_full_size(oracle_mod, tile_env, name, tile):
    tile_env(tile)
    w = W.WORKLOADS[name]
    say("case full-size", name, tile)
    inp = W.make_inputs(w)
    C_bits, info = run_gemm(inp.A, inp.B, w.M, w.N, w.K, w.dtype, w.out, w.layout,
                            scale=(inp.scale_a, inp.scale_b), return_plan_info=True)
    say("  plan", info)
    C = decode(C_bits)
    assert np.all(np.isfinite(C))
    if name in FULL_C:
        C_ref, S = _oracle_full(oracle_mod, name, inp)
        r = assert_within_bound(C, C_ref, S, w.dtype, name)
        say("  whole C (%d entries): worst err/bound %.3g" % (C.size, r))
        return
    rows, cols = block_entries(w.M, w.N, seed=w.seed)
    sigma = oracle_mod.sigma_of(inp.scale_a, inp.scale_b)
    t0 = time.perf_counter()
    c_ref, s = oracle_mod.gemm_bt_entries(inp.A, inp.B, rows, cols, dtype=w.dtype, sigma=sigma)
    say("  oracle: %d entries (one per 16 x 16 block + border rows / columns) in %.1f s" % (
        len(rows), time.perf_counter() - t0))
    r = assert_within_bound(C[rows, cols], c_ref, s, w.dtype, name)
    say("  worst err/bound %.3g" % r)


# ------------------------------------------------------------------ preshuffle kernel

@pytest.mark.parametrize("dtype,N,K", [("bf16", 48, 96), ("bf16", 256, 1056), ("e4m3", 64, 320), ("e4m3", 528, 8256),
                                       ("bf16", 8192, 8192)])
def test_preshuffle_byte_exact(dtype, N, K):
    from oracle import layout as OL
    say("case preshuffle", dtype, N, K)
    rng = np.random.default_rng(N + K)
    code = tg.GEMM_E4M3_OUT_BF16 if dtype == "e4m3" else tg.GEMM_BF16_OUT_BF16
    if dtype == "bf16":
        B = rng.integers(0, 65536, size=(N, K), dtype=np.uint32).astype(np.uint16)
    else:
        B = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    want = OL.preshuffle_b_bytes(B)
    with tg.Plan(64, N, K, code, tg.GEMM_LAYOUT_BT_PRESHUFFLED) as p:
        dB = torch.from_numpy(B.view(np.uint8).reshape(-1).copy()).cuda()
        out = torch.zeros(tg.gemm_preshuffled_b_bytes(p.handle), dtype=torch.uint8, device="cuda")
        p.preshuffle_b(dB.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want)


# ------------------------------------------------------------------ edge cases

def test_k_zero_gives_zeros(tile_env):
    tile_env(None)
    say("case K=0")
    A = np.zeros((0,), np.uint16)
    C = run_gemm(A.reshape(64, 0), np.zeros((0,), np.uint16).reshape(32, 0), 64, 32, 0, "bf16", "bf16", "bt")
    assert np.all(C == 0)


def test_m_zero_is_noop():
    say("case M=0")
    with tg.Plan(0, 64, 64, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        C = torch.full((16,), 7, dtype=torch.uint8, device="cuda")
        p.run(0, 0, C.data_ptr(), None, 0)
        torch.cuda.synchronize()
        assert torch.all(C == 7)


# The kernels whose correctness rests on hand-counted vmcnt immediates and one
# barrier per step, at 4096^3 in the planner's own configuration: 20 runs of
# each must give the same C bit for bit (a race would show as a run that
# differs).  (workload, expected kernel threads)
REPEAT = [("bf16_8192_preshuffled", 512), ("e4m3_8192_preshuffled", 512), ("e4m3_8192", 512),
          ("bf16_4096", 512), ("mxfp4_8192", 512), ("mxfp8_8192", 512), ("i8_8192_bt", 512)]


@pytest.mark.parametrize("name,threads", REPEAT)
def test_repeat_runs_bitwise_stable(tile_env, name, threads):
    tile_env(None)
    M = N = K = 4096
    w = W.WORKLOADS[name]
    say("case repeat x20", name, M, N, K)
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=3)
    code = {"bf16": tg.GEMM_BF16_OUT_BF16, "e4m3": tg.GEMM_E4M3_OUT_BF16, "mxfp4": tg.GEMM_MXFP4_OUT_BF16,
            "mxfp8": tg.GEMM_MXFP8_OUT_BF16, "i8": tg.GEMM_I8_OUT_BF16}[w.dtype]
    s = torch.cuda.current_stream().cuda_stream
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16) if x.dtype == np.uint16
                                     else np.ascontiguousarray(x)).cuda()
    with tg.Plan(M, N, K, code, tg.LAYOUTS[w.layout]) as p:
        info = p.info()
        assert info["tile_m"] == 256 and info["threads"] == threads, info
        A, B = dev(inp.A), dev(inp.B)
        if w.layout == "bt_preshuffled":
            Bs = torch.empty(tg.gemm_preshuffled_b_bytes(p.handle), dtype=torch.uint8, device="cuda")
            p.preshuffle_b(B.data_ptr(), Bs.data_ptr(), s)
            B = Bs
        sc = torch.tensor([inp.scale_a, inp.scale_b], dtype=torch.float32, device="cuda")
        imgs = []
        if w.dtype.startswith("mx"):
            for operand, blocks in ((0, inp.sa_blocks), (1, inp.sb_blocks)):
                src = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
                img = torch.empty(p.bscale_image_bytes(operand), dtype=torch.uint8, device="cuda")
                p.preshuffle_bscale(operand, src.data_ptr(), img.data_ptr(), s)
                imgs.append(img)

        def run(C):
            if imgs:
                p.run_mx(A.data_ptr(), imgs[0].data_ptr(), B.data_ptr(), imgs[1].data_ptr(), C.data_ptr(), stream=s)
            else:
                p.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), sc.data_ptr(), s)
        C0 = torch.empty(M * N, dtype=torch.int16, device="cuda")
        C1 = torch.empty_like(C0)
        run(C0)
        for i in range(20):
            C1.fill_(0x5A5A)
            run(C1)
            torch.cuda.synchronize()
            assert torch.equal(C0, C1), "run %d differs from the first in %d entries" % (
                i + 1, int((C0 != C1).sum()))


def test_side_stream_and_scale_pointer(oracle_mod, tile_env):
    tile_env(None)
    say("case side stream")
    M, N, K = 384, 512, 640
    inp = W.int_inputs(M, N, K, "e4m3", seed=17)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        C_bits = run_gemm(inp.A, inp.B, M, N, K, "e4m3", "bf16", "bt", scale=(4.0, 0.5), stream=st)
    C_ref, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype="e4m3", sigma=2.0, want_s=False)
    assert np.array_equal(C_bits, oracle_mod.round_bf16(C_ref))
