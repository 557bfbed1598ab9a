"""Host-side tests of the C ABI: no GPU work is launched here.

* the library loads and exports every function ``include/tgemm.h`` declares;
* the planner's crd2idx / idx2crd agree with the brute-force oracle and the
  pages' worked examples;
* the pre-shuffle layouts the planner hands to the kernel reproduce the
  oracle's pre-shuffle permutation byte for byte;
* the LDS swizzle is a bijection with the bank properties it claims;
* the XCD-aware raster is a bijection onto the tile grid;
* argument validation rejects what it documents, before any device call.
"""
import ctypes
import itertools
import json
import os
import re

import numpy as np
import pytest

import tiled_gemm_amd as tg
from oracle import layout as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    return tg.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tg.EXPORTS)


def test_crd2idx_matches_brute_force(lib):
    rng = np.random.default_rng(11)
    layouts = [((8, 16), (1, 8)), ((4, 64), (64, 1)), ((3, 5, 7), (35, 7, 1)),
               ((2, 3, 4, 5), (1, 2, 6, 24)), ((4, 4, 2), (9, 1, 40))]
    for _ in range(6):
        r = int(rng.integers(1, 6))
        shape = tuple(int(x) for x in rng.integers(1, 5, size=r))
        stride = tuple(int(x) for x in rng.integers(0, 50, size=r))
        layouts.append((shape, stride))
    for shape, stride in layouts:
        table = OL.brute_force_table(shape, stride)
        for n, crd in enumerate(OL.all_coords(shape)):
            assert tg.gemm_layout_crd2idx(shape, stride, crd) == table[n]


def test_golden_examples_through_the_planner(lib):
    with open(os.path.join(GOLDEN, "layout_examples.json")) as f:
        g = json.load(f)
    for c in g["crd2idx"]:
        assert tg.gemm_layout_crd2idx(c["shape"], c["stride"], c["coord"]) == c["index"]
    for c in g["idx2crd"]:
        assert tg.gemm_layout_idx2crd(c["shape"], c["stride"], c["index"]) == tuple(c["coord"])


def test_crd2idx_rejects_out_of_range(lib):
    with pytest.raises(tg.GemmError):
        tg.gemm_layout_crd2idx((8, 16), (1, 8), (8, 0))


@pytest.mark.parametrize("dtype,N,K", [(tg.GEMM_BF16_OUT_BF16, 32, 64), (tg.GEMM_BF16_OUT_BF16, 48, 96),
                                       (tg.GEMM_E4M3_OUT_BF16, 32, 192), (tg.GEMM_E4M3_OUT_BF16, 16, 64)])
def test_preshuffle_layouts_reproduce_oracle_permutation(lib, dtype, N, K):
    p = tg.Plan(64, N, K, dtype, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
    dst_shape, dst_stride = tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B_SHUF)
    src_shape, src_stride = tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B_SRC)
    assert dst_shape == src_shape
    eb = 1 if dtype == tg.GEMM_E4M3_OUT_BF16 else 2
    kbytes = K * eb
    assert dst_shape == (N // 16, kbytes // 64, 4, 16, 16)
    rng = np.random.default_rng(N + K)
    B = rng.integers(0, 256, size=(N, kbytes), dtype=np.uint8)
    out = np.full(N * kbytes, 0xEE, np.uint8)
    flat = B.reshape(-1)
    seen = set()
    # every 16-byte chunk as the kernel moves it: coordinate -> (src, dst)
    for crd in itertools.product(*[range(s) for s in dst_shape[:4]]):
        c5 = crd + (0,)
        s = tg.gemm_layout_crd2idx(src_shape, src_stride, c5)
        d = tg.gemm_layout_crd2idx(dst_shape, dst_stride, c5)
        out[d:d + 16] = flat[s:s + 16]
        seen.add(d)
    assert len(seen) == N * kbytes // 16
    assert tg.gemm_preshuffled_b_bytes(p.handle) == N * kbytes
    want = OL.preshuffle_b_bytes(B.view(np.uint16) if eb == 2 else B)
    assert np.array_equal(out, want)
    p.close()


def _bank_group(row, phys_chunk):
    """16-byte bank group (of 16) of a chunk in a tile with 128-byte rows, for
    an LDS of 64 four-byte banks (256-byte bank line)."""
    return ((row * 128 + phys_chunk * 16) % 256) // 16


def test_lds_swizzle_bijection_and_banks(lib):
    for row in range(64):
        phys = [tg.gemm_lds_swizzle(row, c) for c in range(8)]
        assert sorted(phys) == list(range(8))
    # MFMA operand read: lane l reads row base + l % 16, chunk cbase + l // 16.
    # A read phase joins a rows-0-7 octet with a rows-8-15 octet (any chunk of
    # the same half); every such pair must touch 16 distinct bank groups.
    for base in range(0, 256, 16):
        for cbase in (0, 4):
            groups = {}
            for q in range(4):
                for half in (0, 1):
                    rows = range(base + 8 * half, base + 8 * half + 8)
                    groups[(q, half)] = [_bank_group(r, tg.gemm_lds_swizzle(r, cbase + q)) for r in rows]
                    assert len(set(groups[(q, half)])) == 8
            for qa in range(4):
                for qb in range(4):
                    both = groups[(qa, 0)] + groups[(qb, 1)]
                    assert len(set(both)) == 16, (base, cbase, qa, qb)
    with pytest.raises(tg.GemmError):
        tg.gemm_lds_swizzle(0, 8)


@pytest.mark.parametrize("M,N,K,dtype,layout", [
    (8192, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED),
    (4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT),
    (300, 272, 96, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT),
    (1000, 4096, 512, tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BT),
    (5000, 3000 // 16 * 16, 64, tg.GEMM_BF16_OUT_F32, tg.GEMM_LAYOUT_BT)])
def test_raster_is_a_bijection(lib, M, N, K, dtype, layout):
    p = tg.Plan(M, N, K, dtype, layout)
    info = p.info()
    tiles = [tg.gemm_tile_of_workgroup(p.handle, wg) for wg in range(info["grid"])]
    assert len(set(tiles)) == info["grid"] == info["tiles_m"] * info["tiles_n"]
    assert all(0 <= a < info["tiles_m"] and 0 <= b < info["tiles_n"] for a, b in tiles)
    # workgroups sharing an XCD (wg % 8) get a contiguous run of the grouped raster
    if info["grid"] >= 64:
        xcd0 = [tiles[w] for w in range(0, info["grid"], 8)][:16]
        rows = {t[0] for t in xcd0}
        assert len(rows) <= max(info["group_m"], 2)
    p.close()


def test_plan_choices(lib, monkeypatch):
    def info(*a):
        with tg.Plan(*a) as p:
            return p.info()
    c = info(256, 256, 256, tg.GEMM_BF16_OUT_F32, tg.GEMM_LAYOUT_BT)
    assert c["kernel"] == 0 and c["out_bytes"] == 4
    c = info(4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT)
    assert (c["tile_m"], c["tile_n"], c["grid"]) == (256, 256, 256)
    # B stored N x K: both operands through LDS, two 64 KiB stages, 8 waves
    assert (c["threads"], c["lds_stages"], c["lds_bytes"]) == (512, 2, 128 * 1024)
    c = info(4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
    assert (c["threads"], c["lds_stages"], c["lds_bytes"]) == (512, 4, 128 * 1024)
    c = info(8192, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
    assert c["lds_bytes"] <= 160 * 1024 and c["grid"] == 1024
    c = info(32, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT)
    assert c["kernel"] == 1 and c["grid"] == 256
    # pre-shuffled B at decode shapes: the skinny kernel with B in registers
    # (2 register stages, LDS for A's ring only)
    for M, dt in ((1, tg.GEMM_BF16_OUT_BF16), (32, tg.GEMM_BF16_OUT_F32), (64, tg.GEMM_E4M3_OUT_BF16)):
        c = info(M, 8192, 8192, dt, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
        assert (c["kernel"], c["grid"], c["tile_n"], c["lds_stages"]) == (1, 256, 32, 2)
        assert c["tile_m"] >= M
    c = info(65, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
    assert c["kernel"] == 0
    # integer decode shapes: int8 with either B layout, W4A8 with B pre-shuffled
    assert info(32, 8192, 8192, tg.GEMM_I8_OUT_BF16, tg.GEMM_LAYOUT_BT)["kernel"] == 1
    assert info(32, 8192, 8192, tg.GEMM_I8_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)["kernel"] == 1
    assert info(32, 8192, 8192, tg.GEMM_W4A8_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)["kernel"] == 1
    assert info(32, 8192, 8192, tg.GEMM_W4A8_OUT_BF16, tg.GEMM_LAYOUT_BT)["kernel"] == 0
    assert info(32, 8192, 8192, tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)["kernel"] == 1
    assert info(32, 8192, 8192, tg.GEMM_MXFP8_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)["kernel"] == 1
    assert info(32, 8192, 8192, tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT)["kernel"] == 0
    c = info(8192, 8192, 8192, tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BT)
    assert c["elem_bytes"] == 1 and c["tile_k_bytes"] % 64 == 0
    assert c["lds_stages"] == 2                      # fp8, B N x K: both operands through LDS
    c = info(8192, 8192, 8192, tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED)
    assert c["lds_stages"] == 4                      # fp8, B pre-shuffled: B in registers
    with tg.Plan(4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, kernel=tg.GEMM_KERNEL_PIPE) as p:
        c = p.info()
    assert (c["threads"], c["lds_stages"]) == (512, 4)
    # every forced family disables the skinny kernel and the 128 x 128 default
    for kc, tile, threads in ((tg.GEMM_KERNEL_GENERIC_128, 128, 256), (tg.GEMM_KERNEL_GENERIC_256, 256, 256),
                              (tg.GEMM_KERNEL_TILE256, 256, 512), (tg.GEMM_KERNEL_PIPE, 256, 512),
                              (tg.GEMM_KERNEL_PIPE4, 256, 256)):
        with tg.Plan(32, 1024, 1024, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT_PRESHUFFLED, kernel=kc) as p:
            c = p.info()
        assert (c["kernel"], c["tile_m"], c["threads"]) == (0, tile, threads), kc


def test_plan_options_are_checked(lib):
    opt = tg.gemm_plan_options(99, 0)
    assert not lib.gemm_plan_create_opt(256, 256, 256, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, ctypes.byref(opt))
    assert "kernel choice" in tg.gemm_last_error()
    opt = tg.gemm_plan_options(0, 65)
    assert not lib.gemm_plan_create_opt(256, 256, 256, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, ctypes.byref(opt))
    # NULL options: exactly gemm_plan_create
    h = lib.gemm_plan_create_opt(4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, None)
    assert h
    a = tg.gemm_plan_query(h)
    lib.gemm_plan_destroy(h)
    with tg.Plan(4096, 4096, 4096, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert p.info() == a
    # a family without a kernel for the dtype / layout is refused
    for dt, lay, kc in ((tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT, tg.GEMM_KERNEL_PIPE),
                        (tg.GEMM_I8_OUT_BF16, tg.GEMM_LAYOUT_BT, tg.GEMM_KERNEL_GENERIC_128),
                        (tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BN, tg.GEMM_KERNEL_PIPE),
                        (tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_AT, tg.GEMM_KERNEL_GENERIC_256)):
        with pytest.raises(tg.GemmError, match="kernel choice"):
            tg.Plan(512, 512, 1024, dt, lay, kernel=kc)


def test_library_reads_no_environment(lib):
    # The planner's choices depend on the arguments alone: the library's
    # imports hold no getenv.
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", tg.LIB_PATH], capture_output=True, text=True).stdout
    assert "getenv" not in out


@pytest.mark.parametrize("args,code", [
    ((16, 16, 64, 7, 0), tg.GEMM_ERR_INVALID_ARG),              # unknown dtype
    ((16, 16, 64, 1, 5), tg.GEMM_ERR_INVALID_ARG),              # unknown layout
    ((-1, 16, 64, 1, 0), tg.GEMM_ERR_INVALID_ARG),              # negative
    ((16, 24, 64, 1, 0), tg.GEMM_ERR_UNSUPPORTED),              # N % 16
    ((16, 16, 40, 1, 0), tg.GEMM_ERR_UNSUPPORTED),              # bf16 K*2 % 64
    ((16, 16, 96, 2, 0), tg.GEMM_ERR_UNSUPPORTED),              # fp8 K % 64
    ((16, 16, 1 << 22, 1, 0), tg.GEMM_ERR_UNSUPPORTED),         # row bytes 2^23
    ((1 << 31, 16, 64, 1, 0), tg.GEMM_ERR_UNSUPPORTED),         # above 2^30
])
def test_plan_create_rejects(lib, args, code):
    h = lib.gemm_plan_create(*args)
    assert not h
    assert tg.gemm_last_error() != ""


def test_run_argument_errors_before_device(lib):
    with tg.Plan(64, 64, 64, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run(p.handle, None, 0x1000, 0x2000, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_run(p.handle, 0x1008, 0x1000000, 0x2000000, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert "aligned" in tg.gemm_last_error()
        # C overlapping A
        assert lib.gemm_run(p.handle, 0x100000, 0x200000, 0x100000, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_b(p.handle, None, 0x1000, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_b(p.handle, 0x1000, 0x1000, None) == tg.GEMM_ERR_INVALID_ARG
    assert lib.gemm_run(None, 0x1000, 0x2000, 0x3000, None, None) == tg.GEMM_ERR_INVALID_ARG
    # M == 0 is a successful no-op that touches no device
    with tg.Plan(0, 64, 64, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run(p.handle, None, None, None, None, None) == tg.GEMM_OK


def test_run_ex_argument_errors_before_device(lib):
    """gemm_run_ex rejects a bad epilogue description before any device work."""
    E = tg.gemm_epilogue_args
    A, B, C = 0x100000, 0x200000, 0x300000
    with tg.Plan(64, 64, 64, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        def run(epi):
            return lib.gemm_run_ex(p.handle, A, B, C, ctypes.byref(epi), None)
        assert run(E(None, None, None, 0, 0, 7)) == tg.GEMM_ERR_INVALID_ARG
        assert "epilogue" in tg.gemm_last_error()
        assert run(E(None, None, None, 2, 0, tg.GEMM_EPI_NONE)) == tg.GEMM_ERR_INVALID_ARG
        assert run(E(None, None, None, 0, 0, tg.GEMM_EPI_BIAS_GELU)) == tg.GEMM_ERR_INVALID_ARG
        assert "bias" in tg.gemm_last_error()
        assert run(E(None, None, 0x400000, 0, 0, tg.GEMM_EPI_NONE)) == tg.GEMM_ERR_INVALID_ARG
        assert run(E(0x400002, None, None, 1, 0, tg.GEMM_EPI_NONE)) == tg.GEMM_ERR_INVALID_ARG
        assert "aligned" in tg.gemm_last_error()
        assert run(E(None, 0x400004, None, 0, 1, tg.GEMM_EPI_NONE)) == tg.GEMM_ERR_INVALID_ARG   # per column: 16 B
        assert run(E(None, None, 0x400008, 0, 0, tg.GEMM_EPI_BIAS)) == tg.GEMM_ERR_INVALID_ARG
        # the plain checks still apply
        assert lib.gemm_run_ex(p.handle, A, B, A, None, None) == tg.GEMM_ERR_INVALID_ARG
    assert lib.gemm_run_ex(None, A, B, C, None, None) == tg.GEMM_ERR_INVALID_ARG
    with tg.Plan(0, 64, 64, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        epi = E(None, None, 0x400000, 0, 0, tg.GEMM_EPI_BIAS_RELU)
        assert lib.gemm_run_ex(p.handle, None, None, None, ctypes.byref(epi), None) == tg.GEMM_OK


def test_epilogue_enum_matches_header():
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "tgemm.h")).read()
    for name, value in [("GEMM_EPI_NONE", 0), ("GEMM_EPI_BIAS", 1), ("GEMM_EPI_BIAS_RELU", 2),
                        ("GEMM_EPI_BIAS_SILU", 3), ("GEMM_EPI_BIAS_GELU", 4)]:
        assert re.search(r"\b%s = %d\b" % (name, value), text), name
        assert getattr(tg, name) == value
    assert ctypes.sizeof(tg.gemm_epilogue_args) == 3 * 8 + 3 * 4 + 4    # 3 pointers, 3 int32, padding


@pytest.mark.parametrize("dtype,bits", [(tg.GEMM_MXFP8_OUT_BF16, 8), (tg.GEMM_MXFP4_OUT_BF16, 4)])
@pytest.mark.parametrize("layout", [tg.GEMM_LAYOUT_BT, tg.GEMM_LAYOUT_BT_PRESHUFFLED])
def test_mx_plans(lib, monkeypatch, dtype, bits, layout):
    for M, N, K in [(8192, 8192, 8192), (32, 4096, 1024), (300, 272, 1152)]:
        with tg.Plan(M, N, K, dtype, layout) as p:
            info = p.info()
            if M <= 64 and layout == tg.GEMM_LAYOUT_BT_PRESHUFFLED:      # decode: the skinny kernel
                assert info["kernel"] == 1 and info["tile_n"] == 32
                assert info["scale_form"] == 0
            else:                            # MX tiles: the 8-wave 32x32x64 kernel, image form 1
                assert info["kernel"] == 0 and info["tile_m"] == 256 and info["threads"] == 512
                assert info["scale_form"] == 1
            assert info["elem_bits"] == bits and info["elem_bytes"] == bits // 8
            assert tg.gemm_preshuffled_b_bytes(p.handle) == N * K * bits // 8
            groups = ((K + 127) // 128 + 3) // 4
            assert p.bscale_image_bytes(0) == (M + 63) // 64 * groups * 1024
            assert p.bscale_image_bytes(1) == (N + 63) // 64 * groups * 1024
            assert p.bscale_image_bytes(2) == 0
    # the 4-wave 16x16x128 kernel reads form 0
    with tg.Plan(300, 272, 1152, dtype, layout, kernel=tg.GEMM_KERNEL_PIPE4) as p:
        assert p.info()["threads"] == 256 and p.info()["scale_form"] == 0
    with pytest.raises(tg.GemmError, match="2\\^31"):
        tg.Plan(64, 1 << 21, 1 << 16, dtype, layout)    # block-scale image past 32-bit offsets
    with tg.Plan(64, 1 << 20, 1 << 14, dtype, layout) as p:
        assert p.bscale_image_bytes(1) < 1 << 31
    with pytest.raises(tg.GemmError):
        tg.Plan(64, 64, 80, dtype, layout)              # K % 32
    if bits == 4:
        with pytest.raises(tg.GemmError):
            tg.Plan(64, 64, 96, dtype, layout)          # K/2 bytes not a multiple of 64


@pytest.mark.parametrize("dtype,b_bits", [(tg.GEMM_I8_OUT_BF16, 8), (tg.GEMM_W4A8_OUT_BF16, 4)])
@pytest.mark.parametrize("layout", [tg.GEMM_LAYOUT_BT, tg.GEMM_LAYOUT_BT_PRESHUFFLED])
def test_int_plans(lib, monkeypatch, dtype, b_bits, layout):
    for M, N, K in [(8192, 8192, 8192), (32, 4096, 1024), (300, 272, 1152), (1, 16, 128)]:
        with tg.Plan(M, N, K, dtype, layout) as p:
            info = p.info()
            skinny = M <= 64 and (b_bits == 8 or layout == tg.GEMM_LAYOUT_BT_PRESHUFFLED)
            if skinny:                       # decode shapes: the skinny kernels
                assert info["kernel"] == 1 and info["tile_n"] == 32 and info["tile_m"] >= M
            else:
                assert info["kernel"] == 0 and info["tile_m"] == 256 and info["threads"] == 512   # 8-wave pipelined
            assert info["elem_bits"] == 8 and info["elem_bytes"] == 1 and info["b_elem_bits"] == b_bits
            assert info["out_bytes"] == 2
            assert tg.gemm_preshuffled_b_bytes(p.handle) == N * K * b_bits // 8
            assert tuple(map(tuple, tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_A))) == ((M, K), (K, 1))
            kb = K * b_bits // 8
            assert tuple(map(tuple, tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B))) == ((N, kb), (kb, 1))
            assert tuple(map(tuple, tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B_SHUF)))[0] == (N // 16, kb // 64, 4, 16, 16)
            assert p.bscale_image_bytes(0) == 0
    with tg.Plan(512, 512, 1024, dtype, layout, kernel=tg.GEMM_KERNEL_PIPE4) as p:
        assert p.info()["threads"] == 256
    with pytest.raises(tg.GemmError):
        tg.Plan(64, 64, 96, dtype, layout)                    # K % 64
    if b_bits == 4:
        with pytest.raises(tg.GemmError):
            tg.Plan(64, 64, 192, dtype, layout)               # K/2 bytes not whole 64-byte steps
    tg.Plan(64, 64, (1 << 17) - 128, dtype, layout).close()   # largest K without int32 overflow
    with pytest.raises(tg.GemmError, match="2\\^17"):
        tg.Plan(64, 64, 1 << 17, dtype, layout)
    with pytest.raises(tg.GemmError):
        tg.Plan(64, 64, 128, dtype + 2, layout)               # past the last dtype


def test_int_run_guards(lib):
    A, B, C = 0x100000, 0x200000, 0x300000
    with tg.Plan(256, 256, 256, tg.GEMM_W4A8_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run_mx(p.handle, A, A, B, B, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_bscale(p.handle, 0, A, B, None) == tg.GEMM_ERR_INVALID_ARG
        # C overlapping B: B has N * K / 2 bytes
        assert lib.gemm_run(p.handle, A, B, B + 256 * 128 - 16, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_b(p.handle, B, B + 256 * 128 - 16, None) == tg.GEMM_ERR_INVALID_ARG


def test_bn_layout_plans(lib, monkeypatch):
    for dtype in (tg.GEMM_BF16_OUT_BF16, tg.GEMM_BF16_OUT_F32):
        # 256 x 256 tiles: 8 waves, both operands staged in LDS (2 stages);
        # 128 x 128: the generic 4-wave tiled kernel
        for M, N, K, tile, threads in [(4096, 4096, 4096, 256, 512), (300, 272, 1056, 128, 256),
                                       (8, 16, 32, 128, 256)]:
            with tg.Plan(M, N, K, dtype, tg.GEMM_LAYOUT_BN) as p:
                info = p.info()
                assert info["kernel"] == 0 and info["tile_m"] == tile and info["threads"] == threads
                assert tg.gemm_preshuffled_b_bytes(p.handle) == 0
                assert tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B) == ((K, 2 * N), (2 * N, 1))
                assert lib.gemm_preshuffle_b(p.handle, 0x100000, 0x200000, None) == tg.GEMM_ERR_INVALID_ARG
        with tg.Plan(4096, 4096, 4096, dtype, tg.GEMM_LAYOUT_BN, kernel=tg.GEMM_KERNEL_GENERIC_256) as p:
            assert p.info()["threads"] == 256                # the generic tiled kernel
    # fp8 e4m3 and int8 with B stored K x N: the LDS-staged kernel on 256 x 256 tiles at every size
    for dtype in (tg.GEMM_E4M3_OUT_BF16, tg.GEMM_I8_OUT_BF16):
        for M, N, K in [(4096, 4096, 4096), (300, 272, 1088), (1, 16, 64)]:
            with tg.Plan(M, N, K, dtype, tg.GEMM_LAYOUT_BN) as p:
                info = p.info()
                assert (info["kernel"], info["tile_m"], info["threads"], info["lds_stages"]) == (0, 256, 512, 2)
                assert tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B) == ((K, N), (N, 1))
                assert tg.gemm_preshuffled_b_bytes(p.handle) == 0
    for dtype in (tg.GEMM_MXFP8_OUT_BF16, tg.GEMM_W4A8_OUT_BF16):
        with pytest.raises(tg.GemmError, match="bf16, fp8 e4m3 and int8"):
            tg.Plan(256, 256, 256, dtype, tg.GEMM_LAYOUT_BN)
    with pytest.raises(tg.GemmError, match="2\\^31"):
        tg.Plan(256, 1 << 16, 1 << 14, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BN)
    with pytest.raises(tg.GemmError):
        tg.Plan(256, 256, 256, tg.GEMM_BF16_OUT_BF16, -1)


def test_at_layout_plans(lib):
    # A stored K x M (B N x K or K x N): always the 8-wave LDS-staged kernel
    # on 256 x 256 tiles, whatever the size
    for layout, b_kn in ((tg.GEMM_LAYOUT_AT, False), (tg.GEMM_LAYOUT_AT_BN, True)):
        for dtype in (tg.GEMM_BF16_OUT_BF16, tg.GEMM_BF16_OUT_F32):
            for M, N, K in [(4096, 4096, 4096), (296, 272, 1056), (8, 16, 32)]:
                with tg.Plan(M, N, K, dtype, layout) as p:
                    info = p.info()
                    assert (info["kernel"], info["tile_m"], info["threads"], info["lds_stages"]) == (0, 256, 512, 2)
                    assert tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_A) == ((K, 2 * M), (2 * M, 1))
                    want_b = ((K, 2 * N), (2 * N, 1)) if b_kn else ((N, 2 * K), (2 * K, 1))
                    assert tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_B) == want_b
                    assert tg.gemm_preshuffled_b_bytes(p.handle) == (0 if b_kn else N * K * 2)
        # 8-bit A stored K x M: the same kernel, 8-bit transpose reads
        for dtype in (tg.GEMM_E4M3_OUT_BF16, tg.GEMM_I8_OUT_BF16):
            for M, N, K in [(4096, 4096, 4096), (304, 272, 1088), (16, 16, 64)]:
                with tg.Plan(M, N, K, dtype, layout) as p:
                    info = p.info()
                    assert (info["kernel"], info["tile_m"], info["threads"]) == (0, 256, 512)
                    assert tg.gemm_plan_layout(p.handle, tg.GEMM_VIEW_A) == ((K, M), (M, 1))
            with pytest.raises(tg.GemmError, match="16-byte"):
                tg.Plan(296, 256, 256, dtype, layout)                     # M bytes % 16
        for dtype in (tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_W4A8_OUT_BF16):
            with pytest.raises(tg.GemmError, match="bf16, fp8 e4m3 and int8"):
                tg.Plan(256, 256, 256, dtype, layout)
        with pytest.raises(tg.GemmError, match="16-byte"):
            tg.Plan(300, 256, 256, tg.GEMM_BF16_OUT_BF16, layout)        # M % 8
        with pytest.raises(tg.GemmError, match="2\\^31"):
            tg.Plan(1 << 16, 256, 1 << 14, tg.GEMM_BF16_OUT_BF16, layout)
    with pytest.raises(tg.GemmError):
        tg.Plan(256, 256, 256, tg.GEMM_BF16_OUT_BF16, 5)


def test_mx_entry_point_guards(lib):
    A, B, C, SA, SB = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    with tg.Plan(256, 256, 256, tg.GEMM_MXFP4_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run(p.handle, A, B, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert "gemm_run_mx" in tg.gemm_last_error()
        assert lib.gemm_run_ex(p.handle, A, B, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_run_mx(p.handle, A, None, B, SB, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_run_mx(p.handle, A, SA + 4, B, SB, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_bscale(p.handle, 2, SA, SB, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_bscale(p.handle, 0, None, SB, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_bscale(p.handle, 0, SA, SA + 8, None) == tg.GEMM_ERR_INVALID_ARG   # misaligned
        assert lib.gemm_preshuffle_bscale(p.handle, 0, SA, SA + 16, None) == tg.GEMM_ERR_INVALID_ARG  # overlap
    with tg.Plan(256, 256, 256, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run_mx(p.handle, A, SA, B, SB, C, None, None) == tg.GEMM_ERR_INVALID_ARG
        assert lib.gemm_preshuffle_bscale(p.handle, 0, SA, SB, None) == tg.GEMM_ERR_INVALID_ARG
        assert p.bscale_image_bytes(0) == 0
    with tg.Plan(0, 256, 256, tg.GEMM_MXFP8_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        assert lib.gemm_run_mx(p.handle, None, None, None, None, None, None, None) == tg.GEMM_OK


def test_split_k_plans(lib, monkeypatch):
    """Split K (gemm_run_ws): slices while 256 x 256 tiles x slices <= 256 and
    each slice keeps >= 8 K steps; every slice non-empty; workspace bytes."""
    forced = {"splits": 0, "kernel": tg.GEMM_KERNEL_AUTO}

    def plan(M, N, K, dt=tg.GEMM_BF16_OUT_BF16, lay=tg.GEMM_LAYOUT_BT_PRESHUFFLED):
        with tg.Plan(M, N, K, dt, lay, **forced) as p:
            return p.info(), p.workspace_bytes()
    for M, want in ((65, 8), (256, 8), (257, 4), (512, 4), (768, 2), (1024, 2), (1025, 1), (8192, 1)):
        info, ws = plan(M, 8192, 8192)
        assert info["ws_splits"] == want, (M, info["ws_splits"])
        assert ws == (want * M * 8192 * 4 if want > 1 else 0)
        tiles = -(-M // 256) * 32
        assert info["ws_grid"] == (tiles * want if want > 1 else info["grid"])
    # K bounds the slices: 8 steps (1 KiB of K) each at least
    assert plan(256, 8192, 2048)[0]["ws_splits"] == 4            # 32 steps of 128 bytes
    assert plan(256, 8192, 512)[0]["ws_splits"] == 1
    # skinny, MX and K-major layouts never split
    assert plan(64, 8192, 8192)[0]["ws_splits"] == 1
    # fp8 splits only where its unsplit plan takes 256 x 256 tiles
    assert plan(256, 8192, 8192, tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BT)[0]["ws_splits"] == 1
    assert plan(1024, 8192, 8192, tg.GEMM_E4M3_OUT_BF16, tg.GEMM_LAYOUT_BT)[0]["ws_splits"] == 2
    assert plan(1024, 8192, 8192, tg.GEMM_E4M3_OUT_BF16)[0]["ws_splits"] == 2
    assert plan(256, 8192, 8192, tg.GEMM_I8_OUT_BF16)[0]["ws_splits"] == 8          # 64 steps of 128 bytes
    assert plan(256, 8192, 8192, tg.GEMM_W4A8_OUT_BF16, tg.GEMM_LAYOUT_BT)[0]["ws_splits"] == 4   # partials <= B
    assert plan(256, 8192, 8192, tg.GEMM_MXFP4_OUT_BF16)[0]["ws_splits"] == 1
    assert plan(256, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BN)[0]["ws_splits"] == 1
    # a forced count, uneven slices; an impossible one is refused (no split)
    forced["splits"] = 3
    assert plan(136, 528, 4160)[0]["ws_splits"] == 3
    assert plan(136, 528, 4160, tg.GEMM_E4M3_OUT_BF16)[0]["ws_splits"] == 3   # forced: fp8 too
    forced["splits"] = 64
    assert plan(136, 528, 4160)[0]["ws_splits"] == 1                # 65 steps: slices would be empty
    # the generic tiled kernel does not read the split fields: never split on it
    forced["splits"] = 4
    forced["kernel"] = tg.GEMM_KERNEL_GENERIC_256
    assert plan(256, 8192, 8192)[0]["ws_splits"] == 1


def test_run_ws_argument_errors(lib):
    M, N, K = 256, 8192, 8192
    with tg.Plan(M, N, K, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT) as p:
        need = p.workspace_bytes()
        A, B, C, Wk = 1 << 32, 2 << 32, 3 << 32, 4 << 32          # never dereferenced: validation fails first
        with pytest.raises(tg.GemmError) as e:
            p.run_ws(A, B, C, Wk + 8, need)
        assert e.value.code == tg.GEMM_ERR_INVALID_ARG and "aligned" in tg.gemm_last_error()
        with pytest.raises(tg.GemmError) as e:
            p.run_ws(A, B, C, C, need)                             # workspace over C
        assert "overlaps" in tg.gemm_last_error()
        with pytest.raises(tg.GemmError) as e:
            p.run_ws(A, B, C, Wk, need, epilogue=tg.GEMM_EPI_BIAS)  # bias epilogue without a bias
        assert e.value.code == tg.GEMM_ERR_INVALID_ARG
    assert tg.gemm_workspace_bytes(None) == 0
