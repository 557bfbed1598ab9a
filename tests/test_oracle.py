"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin is chosen so that a plausible mistake (a dropped term, a sign, a
swapped index, a transposed operand, a wrong decoder bit) fails at least one:
identity and permutation matrices, closed-form rank-1 products, all-ones,
exact rational brute force on tiny non-square shapes, the format definitions
of bf16 / e4m3fn checked against torch's decoders, round-to-nearest-even
ties, and the layout worked examples printed on the FlyDSL pages.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def e4m3(x):
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_matches_torch_on_every_code(oracle_mod):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle_mod.bf16_value(c) for c in codes[::97]])
    w = want[::97]
    nan = np.isnan(w)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], w[~nan])
    for bits, val in [(0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133),
                      (0x7F7F, 3.3895313892515355e38), (0x8000, -0.0)]:
        assert oracle_mod.bf16_value(bits) == val


def test_e4m3fn_decoder_matches_torch_and_format(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle_mod.e4m3fn_value(int(c)) for c in codes])
    nan = np.isnan(want)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # format definition: largest finite 448, smallest subnormal 2^-9, 1.0 = 0 0111 000
    assert oracle_mod.e4m3fn_value(0x7E) == 448.0
    assert oracle_mod.e4m3fn_value(0x01) == 2.0 ** -9
    assert oracle_mod.e4m3fn_value(0x08) == 2.0 ** -6
    assert oracle_mod.e4m3fn_value(0x38) == 1.0
    assert oracle_mod.e4m3fn_value(0xB8) == -1.0


# ---------------------------------------------------------------- rounding

def test_round_bf16_golden_ties(oracle_mod):
    with open(os.path.join(GOLDEN, "bf16_rounding.json")) as f:
        cases = json.load(f)["cases"]
    xs = np.array([c["x"] for c in cases])
    got = oracle_mod.round_bf16(xs)
    for c, g in zip(cases, got):
        assert int(g) == int(c["bits"], 16), c
        assert oracle_mod.bf16_value(int(g)) == c["value"]


def test_round_bf16_matches_torch_on_fp32_values(oracle_mod):
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 1000,
                        rng.standard_normal(2000).astype(np.float32) * 1e-30,
                        np.float32([1e-39, -3e-40, 65504.5, 3.38e38])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle_mod.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- the GEMM

def test_identity(oracle_mod):
    rng = np.random.default_rng(1)
    K = 24
    B = bf16(rng.integers(-8, 9, size=(10, K)))
    I = bf16(np.eye(K))
    C, S = oracle_mod.gemm_bt(I, B)          # A = I  =>  C = B^T
    Bv = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(C, Bv.T)
    assert np.array_equal(S, np.abs(Bv.T))
    A = bf16(rng.integers(-8, 9, size=(7, K)))
    C2, _ = oracle_mod.gemm_bt(A, I)         # B = I  =>  C = A
    Av = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(C2, Av)


def test_permutation(oracle_mod):
    rng = np.random.default_rng(2)
    K, N = 9, 5
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), perm] = 1.0              # row i selects k = perm[i]
    Bf = rng.integers(-5, 6, size=(N, K)).astype(np.float32)
    C, _ = oracle_mod.gemm_bt(bf16(P), bf16(Bf))
    assert np.array_equal(C, Bf[:, perm].T.astype(np.float64))


def test_rank1_closed_form(oracle_mod):
    u = np.array([1, -2, 3], np.float32)
    v = np.array([2, 1, -1, 4, 0], np.float32)
    x = np.array([1, 2, -3, 1, 1, -1, 2], np.float32)
    y = np.array([-1, 1, 1, 2, -2, 3, 1], np.float32)
    A = np.outer(u, x)
    B = np.outer(v, y)
    C, S = oracle_mod.gemm_bt(bf16(A), bf16(B))
    xy = float(np.dot(x.astype(np.float64), y))
    assert np.array_equal(C, np.outer(u, v).astype(np.float64) * xy)
    assert np.array_equal(S, np.abs(np.outer(u, v)).astype(np.float64) * float(np.abs(x * y).sum()))


def test_all_ones_and_alternating(oracle_mod):
    K = 33
    ones = bf16(np.ones((4, K)))
    C, S = oracle_mod.gemm_bt(ones, bf16(np.ones((6, K))))
    assert np.all(C == K) and np.all(S == K)
    alt = bf16(np.tile((-1.0) ** np.arange(K), (4, 1)))
    C, S = oracle_mod.gemm_bt(alt, bf16(np.ones((3, K))))
    assert np.all(C == 1.0) and np.all(S == K)   # K odd: one uncancelled +1


@pytest.mark.parametrize("M,N,K", [(4, 4, 4), (3, 5, 7), (5, 2, 6)])
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_brute_force_rational(oracle_mod, M, N, K, dtype):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 3).astype(np.float32)
    if dtype == "bf16":
        A, B = bf16(a), bf16(b)
        table = torch.from_numpy(np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.int16)) \
            .view(torch.bfloat16).double().numpy()
        dec = lambda bits: Fraction(float(table[int(bits)]))
        sa, sb = 1.0, 1.0
    else:
        A, B = e4m3(a), e4m3(b)
        table = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
        dec = lambda bits: Fraction(float(table[int(bits)]))
        sa, sb = 0.375, 1.5
    sigma = oracle_mod.sigma_of(sa, sb)
    C, S = oracle_mod.gemm_bt(A, B, dtype=dtype, sigma=sigma)
    for i in range(M):
        for j in range(N):
            exact = sum(dec(A[i, k]) * dec(B[j, k]) for k in range(K)) * Fraction(sa) * Fraction(sb)
            mag = sum(abs(dec(A[i, k]) * dec(B[j, k])) for k in range(K)) * Fraction(sa) * Fraction(sb)
            assert C[i, j] == float(exact), (i, j)   # small sums are exact in fp64
            assert S[i, j] == float(mag), (i, j)


def test_entries_equal_full(oracle_mod):
    inp = workloads.make_inputs(workloads.WORKLOADS["bf16_4096"], M=40, N=24, K=64, seed=5)
    C, S = oracle_mod.gemm_bt(inp.A, inp.B)
    rows = np.array([0, 39, 17, 5, 39])
    cols = np.array([23, 0, 11, 5, 23])
    c, s = oracle_mod.gemm_bt_entries(inp.A, inp.B, rows, cols)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_entries_reject_out_of_range(oracle_mod):
    inp = workloads.int_inputs(4, 4, 64, "bf16", 1)
    with pytest.raises(IndexError):
        oracle_mod.gemm_bt_entries(inp.A, inp.B, [4], [0])


# ---------------------------------------------------------------- layouts

def test_layout_golden_examples():
    with open(os.path.join(GOLDEN, "layout_examples.json")) as f:
        g = json.load(f)
    for c in g["crd2idx"]:
        assert L.crd2idx(tuple(c["coord"]), tuple(c["shape"]), tuple(c["stride"])) == c["index"]
    for c in g["idx2crd"]:
        assert L.idx2crd(c["index"], tuple(c["shape"]), tuple(c["stride"])) == tuple(c["coord"])


def test_layout_brute_force_table():
    # compact column-major: the table is 0..size-1 in order
    assert np.array_equal(L.brute_force_table((8, 16), (1, 8)), np.arange(128))
    # row-major (4,6):(6,1) visited colexicographically
    t = L.brute_force_table((4, 6), (6, 1))
    assert list(t[:5]) == [0, 6, 12, 18, 1]
    # nested shapes flatten
    assert L.crd2idx(((1, 2), 3), ((2, 4), 5), ((1, 2), 8)) == 1 + 4 + 24
    # integer coordinates split colexicographically
    assert L.crd2idx(43, (8, 16), (1, 8)) == 43
    assert L.crd2idx(5, (2, 3), (3, 1)) == 1 * 3 + 2 * 1


def test_preshuffle_two_formulations_agree():
    rng = np.random.default_rng(3)
    N, K = 48, 96                                  # bf16: 192 bytes per row
    B = rng.integers(0, 65535, size=(N, K), dtype=np.uint16)
    shuf = L.preshuffle_b_bytes(B)
    raw = B.view(np.uint8).reshape(N, -1)
    kbytes = raw.shape[1]
    assert sorted(shuf.tolist()) == sorted(raw.reshape(-1).tolist())
    for n in range(N):
        for kb in range(kbytes):
            assert shuf[L.preshuffle_src_offset(n, kb, N, kbytes)] == raw[n, kb]
    # a hand-computed element: n=17, byte 70 of a 128-byte row
    assert L.preshuffle_src_offset(17, 70, 32, 128) == ((((1 * 2 + 1) * 4 + 0) * 16 + 1) * 16 + 6)


def test_preshuffle_block_is_one_wave_operand():
    """Each 1 KiB block holds, for lane l = 16*q + r, the 16 bytes of row
    16*nb + r at k-bytes 64*kb + 16*q: one 16-byte load per lane."""
    N, K = 32, 64                                  # bf16 -> 128 bytes per row
    B = (np.arange(N * K, dtype=np.uint32) % 65521).astype(np.uint16).reshape(N, K)
    shuf = L.preshuffle_b_bytes(B).reshape(N // 16, 2, 64, 16)
    raw = B.view(np.uint8).reshape(N, -1)
    for nb in range(N // 16):
        for kb in range(2):
            for lane in range(64):
                q, r = divmod(lane, 16)
                assert np.array_equal(shuf[nb, kb, lane], raw[16 * nb + r, 64 * kb + 16 * q:64 * kb + 16 * q + 16])


def test_preshuffle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        L.preshuffle_b_bytes(np.zeros((24, 64), np.uint16))
    with pytest.raises(ValueError):
        L.preshuffle_b_bytes(np.zeros((32, 40), np.uint8))


# ---------------------------------------------------------------- epilogue
# Pins of oracle.epilogue: identities of the activations that do not restate
# their formulas, values of the standard normal CDF and of e from tables and
# math constants, and linearity against pre-scaled GEMM inputs.

# Phi(z) to 16 digits, from a standard normal table.
PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -1.0: 0.15865525393145707, 0.5: 0.6914624612740131}


def _act(oracle_mod, z, kind):
    z = np.asarray(z, np.float64).reshape(1, -1)
    return oracle_mod.epilogue(z, bias=np.zeros(z.shape[1]), kind=kind)[0]


def test_epilogue_relu_closed_form(oracle_mod):
    z = np.array([-3.0, -0.0, 0.0, 1e-300, 2.5, -1e-300])
    y = _act(oracle_mod, z, "bias_relu")
    assert np.array_equal(y, [0.0, 0.0, 0.0, 1e-300, 2.5, 0.0])
    assert not np.signbit(y).any()           # +0 for every z <= 0


def test_epilogue_gelu_is_z_phi_z(oracle_mod):
    for z, phi in PHI.items():
        assert _act(oracle_mod, [z], "bias_gelu")[0] == pytest.approx(z * phi, rel=1e-14)
    # the tanh approximation differs by ~1.5e-4 at z = 1: must not be what is computed
    assert abs(_act(oracle_mod, [1.0], "bias_gelu")[0] - 0.8411919906082768) > 1e-4


def test_epilogue_silu_values(oracle_mod):
    e = np.e
    assert _act(oracle_mod, [1.0], "bias_silu")[0] == pytest.approx(e / (1 + e), rel=1e-15)
    assert _act(oracle_mod, [0.0], "bias_silu")[0] == 0.0
    # far tails: z * logistic(z) -> z for large z, -> z e^z for very negative z
    assert _act(oracle_mod, [40.0], "bias_silu")[0] == pytest.approx(40.0, rel=1e-15)
    assert _act(oracle_mod, [-800.0], "bias_silu")[0] == 0.0 or abs(_act(oracle_mod, [-800.0], "bias_silu")[0]) < 1e-300
    assert _act(oracle_mod, [-30.0], "bias_silu")[0] == pytest.approx(-30.0 * np.exp(-30.0), rel=1e-12)


@pytest.mark.parametrize("kind", ["bias_silu", "bias_gelu"])
def test_epilogue_odd_part_identity(oracle_mod, kind):
    # logistic(z) + logistic(-z) = 1 and Phi(z) + Phi(-z) = 1 give
    # act(z) - act(-z) = z for both SiLU and GELU.
    z = np.linspace(-12, 12, 97)
    d = _act(oracle_mod, z, kind) - _act(oracle_mod, -z, kind)
    assert np.allclose(d, z, rtol=0, atol=1e-13)


def test_epilogue_order_scales_bias_then_activation(oracle_mod):
    acc = np.array([[-1.0, 3.0], [2.0, -4.0]])
    sa = np.array([2.0, -1.0])        # per row
    sb = np.array([1.0, 0.5])         # per column
    bias = np.array([3.0, -1.0])
    # z = (acc * sa[m]) * sb[n] + bias[n], worked by hand
    z = np.array([[-2.0 + 3.0, 3.0 - 1.0], [-2.0 + 3.0, 2.0 - 1.0]])
    assert np.array_equal(oracle_mod.epilogue(acc, sa, sb, bias, "bias"), z)
    assert np.array_equal(oracle_mod.epilogue(acc, sa, sb, bias, "bias_relu"), np.maximum(z, 0))
    # ReLU after the bias, not before: relu(acc) + bias would give [3, 3.5] in row 0
    assert oracle_mod.epilogue(acc, sa, sb, bias, "bias_relu")[0, 0] == 1.0
    # scalar scales broadcast; "none" ignores the bias
    assert np.array_equal(oracle_mod.epilogue(acc, 2.0, 0.5, None, "none"), acc)


def test_epilogue_scale_vectors_equal_prescaled_inputs(oracle_mod):
    # Per-row s_a scales row m of A, per-column s_b scales row n of B: with
    # powers of two the pre-scaled bf16 inputs are exact, so the GEMM of the
    # scaled inputs must equal the epilogue applied to the unscaled GEMM.
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 64
    a = rng.integers(-4, 5, (M, K)).astype(np.float32)
    b = rng.integers(-4, 5, (N, K)).astype(np.float32)
    sa = 2.0 ** rng.integers(-3, 4, M)
    sb = 2.0 ** rng.integers(-3, 4, N)
    acc, _ = oracle_mod.gemm_bt(bf16(a), bf16(b), dtype="bf16")
    scaled, _ = oracle_mod.gemm_bt(bf16(a * sa[:, None].astype(np.float32)), bf16(b * sb[:, None].astype(np.float32)),
                                   dtype="bf16")
    assert np.array_equal(oracle_mod.epilogue(acc, sa, sb, None, "none"), scaled)
    bias = rng.integers(-8, 9, N).astype(np.float64)
    assert np.array_equal(oracle_mod.epilogue(acc, sa, sb, bias, "bias") - bias[None, :], scaled)


def test_epilogue_rejects_unknown_kind(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.epilogue(np.zeros((1, 1)), kind="bias_tanh")


# ---------------------------------------------------------------- MX operands
# OCP Microscaling formats: E2M1 element values and E8M0 scales as the format
# definitions list them; the MX GEMM against an exact rational brute force
# whose element packing (even element in the low nibble) and scale placement
# (one scale per 32 elements along K) are written independently here.

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decoder_table(oracle_mod):
    for code in range(16):
        mag = E2M1_TABLE[code & 7]
        assert oracle_mod.e2m1_value(code) == (-mag if code & 8 else mag)


def test_e8m0_decoder(oracle_mod):
    assert oracle_mod.e8m0_value(127) == 1.0
    assert oracle_mod.e8m0_value(128) == 2.0
    assert oracle_mod.e8m0_value(126) == 0.5
    assert oracle_mod.e8m0_value(0) == 2.0 ** -127
    assert oracle_mod.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle_mod.e8m0_value(255))


def _mx_random(rng, rows, K, fmt):
    """Random codes and scales, plus their exact rational values."""
    if fmt == "mxfp8":
        codes = rng.integers(0, 256, (rows, K)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x38                  # no NaN codes
        vals = [[Fraction(float(torch.tensor(int(c), dtype=torch.uint8).view(torch.float8_e4m3fn).float()))
                 for c in r] for r in codes]
        packed = codes
    else:
        codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
        vals = [[Fraction(-E2M1_TABLE[c & 7] if c & 8 else E2M1_TABLE[c & 7]) for c in r] for r in codes]
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(120, 135, (rows, K // 32)).astype(np.uint8)
    exact = [[vals[i][k] * Fraction(2) ** (int(scales[i][k // 32]) - 127) for k in range(K)] for i in range(rows)]
    return packed, scales, exact


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (2, 4, 96)])
def test_mx_brute_force_rational(oracle_mod, fmt, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + len(fmt))
    A, SA, ea = _mx_random(rng, M, K, fmt)
    B, SB, eb = _mx_random(rng, N, K, fmt)
    C, S = oracle_mod.gemm_bt_mx(A, SA, B, SB, K, fmt)
    for i in range(M):
        for j in range(N):
            want = sum(ea[i][k] * eb[j][k] for k in range(K))
            assert C[i, j] == float(want)
            assert S[i, j] == float(sum(abs(ea[i][k] * eb[j][k]) for k in range(K)))
    rows, cols = np.array([0, M - 1, 1]), np.array([N - 1, 0, 2])
    Ce, Se = oracle_mod.gemm_bt_mx_entries(A, SA, B, SB, K, rows, cols, fmt)
    assert np.array_equal(Ce, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_mxfp8_with_unit_scales_is_the_e4m3_gemm(oracle_mod):
    rng = np.random.default_rng(3)
    A = e4m3(rng.normal(0, 2, (6, 128)))
    B = e4m3(rng.normal(0, 2, (7, 128)))
    ones_a = np.full((6, 4), 127, np.uint8)
    ones_b = np.full((7, 4), 127, np.uint8)
    C, _ = oracle_mod.gemm_bt_mx(A, ones_a, B, ones_b, 128, "mxfp8")
    R, _ = oracle_mod.gemm_bt(A, B, dtype="e4m3")
    assert np.array_equal(C, R)


def test_mxfp4_nibble_order_and_block_of_scale(oracle_mod):
    # one nonzero element in A at k = 33 (high nibble of byte 16, scale block 1)
    K = 64
    A = np.zeros((1, K // 2), np.uint8)
    A[0, 16] = 0x2 << 4                      # element 33 = code 2 = 1.0
    SA = np.array([[127, 129]], np.uint8)     # block 1 scaled by 4
    B = np.zeros((1, K // 2), np.uint8)
    B[0, 16] = 0x7 << 4                      # element 33 = 6.0
    SB = np.array([[127, 127]], np.uint8)
    C, _ = oracle_mod.gemm_bt_mx(A, SA, B, SB, K, "mxfp4")
    assert C[0, 0] == 24.0
    with pytest.raises(ValueError):
        oracle_mod.gemm_bt_mx(A, SA[:, :1], B, SB, K, "mxfp4")


def test_bscale_image_hand_computed_entries():
    # R = 70 rows, K = 256: 8 blocks per row, 2 K-slices -> 1 group; 2 row quads.
    S = (np.arange(70 * 8) % 251).astype(np.uint8).reshape(70, 8)
    img = L.bscale_image(S, 256).reshape(2, 1, 64, 4, 4)
    # quad 1, group 0, lane 17 (row 1 of a block, lane group 1), block 0, slice 1:
    # row 64 + 0 + 1 = 65, K block 4 * (0 + 1) + 1 = 5
    assert img[1, 0, 17, 0, 1] == S[65, 5]
    # quad 0, lane 63 (row 15, group 3), block 2, slice 0: row 47, K block 3
    assert img[0, 0, 63, 2, 0] == S[47, 3]
    # slices 2 and 3 lie past K (only 2 slices): unit scale 127
    assert (img[:, :, :, :, 2:] == 127).all()
    # rows 70.. of quad 1 (block 0 lanes with l % 16 >= 6) are padding
    assert img[1, 0, 6, 0, 0] == 127 and img[1, 0, 5, 0, 0] == S[69, 0]


def test_bscale_image_32_consumer_view():
    # Form 1 from the reader's side: lane l of the 32x32x64 MFMA, row half u
    # of a quad and 64-element slice s' (0..7) of a 512-element group needs
    # the scale of row 32 u + l % 32 for K block 2 s' + l // 32, and reads it
    # from word 2 u + s' % 2, byte s' // 2 of its 16 bytes.  R = 100 rows and
    # K = 640 (20 blocks, 2 groups, the second one partial): every in-range
    # scale appears exactly once and the rest is the unit scale 127.
    R, K = 100, 640
    S = (np.arange(R * (K // 32)) * 7 % 251).astype(np.uint8).reshape(R, K // 32)
    img = L.bscale_image_32(S, K).reshape(2, 2, 64, 4, 4)
    seen = np.zeros(img.shape, bool)
    for quad in range(2):
        for g in range(2):
            for lane in range(64):
                for u in range(2):
                    for sp in range(8):
                        row = 64 * quad + 32 * u + lane % 32
                        blk = 16 * g + 2 * sp + lane // 32
                        pos = (quad, g, lane, 2 * u + sp % 2, sp // 2)
                        seen[pos] = True
                        want = S[row, blk] if row < R and blk < K // 32 else 127
                        assert img[pos] == want, (pos, row, blk)
    assert seen.all()
    # hand-computed: quad 1, group 1, lane 37 (row 5 of the half, K half 1),
    # word 3 (half 1, odd slice), byte 2 -> slice 5: row 64 + 32 + 5 = 101 is
    # past R; lane 37 of word 1 instead: row 69, block 16 + 10 + 1 = 27 past K;
    # byte 0 of word 1 -> slice 1: block 16 + 2 + 1 = 19
    assert img[1, 1, 37, 3, 2] == 127
    assert img[1, 1, 37, 1, 2] == 127
    assert img[1, 1, 37, 1, 0] == S[69, 19]
    # the two forms hold the same bytes, permuted
    assert np.array_equal(np.sort(img.reshape(-1)), np.sort(L.bscale_image(S, K)))


# ---------------------------------------------------------------------------
# Integer operands (int8 A; int8 or packed int4 B)
# ---------------------------------------------------------------------------
INT4_TABLE = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_int_decoder_tables(oracle_mod):
    assert [oracle_mod.int4_value(n) for n in range(16)] == INT4_TABLE
    assert oracle_mod.int8_value(0x00) == 0 and oracle_mod.int8_value(0x7F) == 127
    assert oracle_mod.int8_value(0x80) == -128 and oracle_mod.int8_value(0xFF) == -1
    assert oracle_mod.int8_value(0x9C) == -100


def _int_random(rng, rows, K, bits):
    """Random bytes and their values decoded independently of the oracle."""
    if bits == 8:
        b = rng.integers(0, 256, (rows, K)).astype(np.uint8)
        vals = [[int(v) - 256 if v >= 128 else int(v) for v in r] for r in b]
        return b, vals
    nib = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    vals = [[INT4_TABLE[int(v)] for v in r] for r in nib]
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), vals


@pytest.mark.parametrize("fmt", ["i8", "w4a8"])
@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (2, 4, 6), (1, 1, 2)])
def test_int_brute_force(oracle_mod, fmt, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + len(fmt))
    A, va = _int_random(rng, M, K, 8)
    B, vb = _int_random(rng, N, K, 8 if fmt == "i8" else 4)
    C, S = oracle_mod.gemm_bt_int(A, B, K, fmt)
    for i in range(M):
        for j in range(N):
            assert C[i, j] == sum(va[i][k] * vb[j][k] for k in range(K))
            assert S[i, j] == sum(abs(va[i][k] * vb[j][k]) for k in range(K))
    rows, cols = np.array([0, M - 1]), np.array([N - 1, 0])
    Ce, Se = oracle_mod.gemm_bt_int_entries(A, B, K, rows, cols, fmt)
    assert np.array_equal(Ce, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_w4a8_nibble_order(oracle_mod):
    # byte 0x21: element 0 = 1 (low nibble), element 1 = 2 (high nibble)
    A = np.array([[10, 100]], np.uint8)
    B = np.array([[0x21]], np.uint8)
    C, _ = oracle_mod.gemm_bt_int(A, B, 2, "w4a8")
    assert C[0, 0] == 10 * 1 + 100 * 2
    # 0xF8: element 0 = -8, element 1 = -1
    C, _ = oracle_mod.gemm_bt_int(A, np.array([[0xF8]], np.uint8), 2, "w4a8")
    assert C[0, 0] == 10 * -8 + 100 * -1


def test_int_extremes_closed_form(oracle_mod):
    K = 4096
    A = np.full((2, K), 0x80, np.uint8)                  # -128
    C, S = oracle_mod.gemm_bt_int(A, np.full((3, K), 0x80, np.uint8), K, "i8")
    assert np.all(C == K * 16384) and np.all(S == K * 16384)
    C, _ = oracle_mod.gemm_bt_int(A, np.full((3, K // 2), 0x88, np.uint8), K, "w4a8")   # -8, -8
    assert np.all(C == K * 1024)
    C, _ = oracle_mod.gemm_bt_int(A, np.full((3, K), 0x7F, np.uint8), K, "i8")
    assert np.all(C == -K * 128 * 127)


def test_int8_agrees_with_the_bf16_gemm_on_exact_values(oracle_mod):
    # every int8 value is exact in bf16 and every partial sum here is exact
    # in fp64, so the float oracle must give the same numbers
    rng = np.random.default_rng(11)
    A = rng.integers(0, 256, (5, 96)).astype(np.uint8)
    B = rng.integers(0, 256, (7, 96)).astype(np.uint8)
    C, S = oracle_mod.gemm_bt_int(A, B, 96, "i8")
    as_bf16 = lambda x: bf16(x.view(np.int8).astype(np.float32))
    R, RS = oracle_mod.gemm_bt(as_bf16(A), as_bf16(B), dtype="bf16")
    assert np.array_equal(C, R) and np.array_equal(S, RS)


def test_int_rejects_bad_shapes(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.gemm_bt_int(np.zeros((2, 64), np.uint8), np.zeros((2, 64), np.uint8), 64, "w4a8")
    with pytest.raises(ValueError):
        oracle_mod.gemm_bt_int(np.zeros((2, 64), np.uint8), np.zeros((2, 32), np.uint8), 64, "i8")
    with pytest.raises(ValueError):
        oracle_mod.gemm_bt_int(np.zeros((2, 64), np.uint8), np.zeros((2, 64), np.uint8), 64, "i4")


# ---------------------------------------------------------------------------
# B stored K x N
# ---------------------------------------------------------------------------
def test_gemm_ab_is_the_plain_matrix_product(oracle_mod):
    # integer values: every sum exact; numpy's int64 matmul is an independent
    # definition of C = A @ B with B as K x N (non-square, so a transposed
    # operand would not even have the right shape)
    rng = np.random.default_rng(21)
    a = rng.integers(-9, 10, (5, 24))
    b = rng.integers(-9, 10, (24, 7))
    C, S = oracle_mod.gemm_ab(bf16(a.astype(np.float32)), bf16(b.astype(np.float32)))
    assert C.shape == (5, 7)
    assert np.array_equal(C, (a @ b).astype(np.float64))
    assert np.array_equal(S, (np.abs(a) @ np.abs(b)).astype(np.float64))
    rows, cols = np.array([0, 4, 2]), np.array([6, 0, 3])
    Ce, Se = oracle_mod.gemm_ab_entries(bf16(a.astype(np.float32)), bf16(b.astype(np.float32)), rows, cols)
    assert np.array_equal(Ce, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_gemm_ab_unit_vectors(oracle_mod):
    # A = e_1 picks row 1 of B: C[0][n] = B[1][n]
    K, N = 4, 6
    a = np.zeros((1, K), np.float32)
    a[0, 1] = 1.0
    b = np.arange(K * N, dtype=np.float32).reshape(K, N)
    C, _ = oracle_mod.gemm_ab(bf16(a), bf16(b))
    assert np.array_equal(C[0], b[1].astype(np.float64))


# ---------------------------------------------------------------------------
# A stored K x M
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b_kn", [False, True])
def test_gemm_at_is_the_plain_matrix_product(oracle_mod, b_kn):
    # integer values: every sum exact; numpy's int64 matmul of the stored
    # arrays is an independent definition: C = A_km^T @ B^T (B N x K) or
    # A_km^T @ B (B K x N).  Non-square, so a wrongly oriented operand would
    # not even have the right shape.
    rng = np.random.default_rng(23)
    M, N, K = 5, 7, 24
    a_km = rng.integers(-9, 10, (K, M))
    b = rng.integers(-9, 10, (K, N) if b_kn else (N, K))
    want = a_km.T @ (b if b_kn else b.T)
    C, S = oracle_mod.gemm_at(bf16(a_km.astype(np.float32)), bf16(b.astype(np.float32)), b_kn=b_kn)
    assert C.shape == (M, N)
    assert np.array_equal(C, want.astype(np.float64))
    assert np.array_equal(S, (np.abs(a_km.T) @ np.abs(b if b_kn else b.T)).astype(np.float64))
    rows, cols = np.array([0, 4, 2]), np.array([6, 0, 3])
    Ce, Se = oracle_mod.gemm_at_entries(bf16(a_km.astype(np.float32)), bf16(b.astype(np.float32)), rows, cols,
                                        b_kn=b_kn)
    assert np.array_equal(Ce, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_gemm_at_unit_vectors(oracle_mod):
    # A stored K x M with column m holding e_{sel[m]}: row m of C is column
    # sel[m] of B^T, i.e. C[m][n] = B[n][sel[m]]
    K, M, N = 6, 3, 5
    sel = [4, 0, 2]
    a_km = np.zeros((K, M), np.float32)
    for m, k in enumerate(sel):
        a_km[k, m] = 1.0
    b = np.arange(N * K, dtype=np.float32).reshape(N, K)
    C, _ = oracle_mod.gemm_at(bf16(a_km), bf16(b))
    for m, k in enumerate(sel):
        assert np.array_equal(C[m], b[:, k].astype(np.float64))
