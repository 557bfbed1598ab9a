"""Seeded synthetic workloads for the tiled GEMM C = A * B^T.

This module only draws inputs: it holds none of the GEMM's arithmetic and is
shared by the tests, the benchmark and the smoke check.  Both the HIP path and
the CPU oracle consume exactly the arrays returned here.

Recipe (every array is raw element bits in row-major order):

* One ``numpy.random.Generator(PCG64(seed))`` per workload; A is drawn first,
  then B.  Samples are float32.
* "integers uniform in [-4, 4]": inclusive integers, ``rng.integers(-4, 5)``.
* "N(mu, sd)": ``rng.standard_normal`` (float32) times sd plus mu;
  "U(lo, hi)": ``rng.random`` (float32, [0, 1)) scaled to [lo, hi).
* bf16: float32 sample rounded to bf16 (nearest-even) by torch's CPU cast.
* e4m3 (OCP e4m3fn): per-tensor scale s = float32(amax(|X|) / 448), then
  q = e4m3fn(clamp(X / s, -448, 448)) by torch's CPU cast; the scale pair is
  returned so that C = (acc * s_a) * s_b.
* MX (OCP Microscaling, block size 32 along K): per block, the E8M0 scale
  exponent is floor(log2(amax)) - emax (emax 8 for e4m3, 2 for e2m1; 2^-127
  for an all-zero block), and each element is X / 2^exp rounded to the
  element format (nearest, ties to even, saturating).  MXFP4 packs two
  elements per byte, the even one in the low nibble.
* int8 / W4A8 (int8 A, packed int4 B): symmetric absmax quantisation per row
  of A and per row of B (one output channel of C): s = float32(amax / 127)
  (int8) or float32(amax / 7) (int4), q = clip(rint(X / s), -127, 127) or
  (-7, 7).  int4 packs two values per byte, the even element in the low
  nibble.  The per-row scales are returned as vectors for the epilogue,
  C = (acc * s_a[row]) * s_b[col].

A is M x K, B is N x K (K contiguous in both), C is M x N.  Layout "bn"
stores B as K x N (N contiguous): it is drawn N x K as above and stored
transposed.  Layouts "at" and "at_bn" store A as K x M the same way (and
"at_bn" B as K x N).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # "bf16", "e4m3", "mxfp8", "mxfp4", "i8" or "w4a8" (int8 A, int4 B)
    out: str            # "f32" or "bf16"
    layout: str         # "bt" (B as N x K), "bt_preshuffled", "bn" (B as K x N), "at" (A as
                        # K x M, B N x K) or "at_bn" (A as K x M, B K x N)
    dist_a: tuple
    dist_b: tuple
    seed: int
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> float:
        """Bytes per element of A."""
        return {"bf16": 2, "e4m3": 1, "mxfp8": 1, "mxfp4": 0.5, "i8": 1, "w4a8": 1}[self.dtype]

    @property
    def b_elem_bytes(self) -> float:
        return 0.5 if self.dtype == "w4a8" else self.elem_bytes

    @property
    def out_bytes(self) -> int:
        return 4 if self.out == "f32" else 2

    @property
    def min_bytes(self) -> int:
        """Each operand read once and C written once."""
        if self.dtype.startswith("mx"):
            scales = (self.M + self.N) * (self.K // 32)
        elif self.dtype in ("i8", "w4a8"):
            scales = (self.M + self.N) * 4              # fp32 per-row / per-column scale vectors
        else:
            scales = 0
        return (int(self.M * self.K * self.elem_bytes + self.N * self.K * self.b_elem_bytes) + scales
                + self.M * self.N * self.out_bytes)


WORKLOADS = {
    "bf16_int_256": Workload("bf16_int_256", 256, 256, 256, "bf16", "f32", "bt",
                             ("int", -4, 4), ("int", -4, 4), 1001,
                             "integer-valued, exact in fp32: bit-exact check"),
    "bf16_4096": Workload("bf16_4096", 4096, 4096, 4096, "bf16", "bf16", "bt",
                          ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1002),
    "bf16_8192_preshuffled": Workload("bf16_8192_preshuffled", 8192, 8192, 8192, "bf16", "bf16",
                                      "bt_preshuffled", ("uniform", -1.0, 1.0),
                                      ("uniform", -1.0, 1.0), 1003),
    "bf16_skinny_32x8192x8192": Workload("bf16_skinny_32x8192x8192", 32, 8192, 8192, "bf16",
                                         "bf16", "bt", ("normal", 0.0, 1.0),
                                         ("normal", 0.0, 0.02), 1004,
                                         "decode-like, HBM-bound"),
    "bf16_skinny_32x8192x8192_preshuffled": Workload("bf16_skinny_32x8192x8192_preshuffled", 32, 8192, 8192,
                                                     "bf16", "bf16", "bt_preshuffled", ("normal", 0.0, 1.0),
                                                     ("normal", 0.0, 0.02), 1014,
                                                     "decode-like with a pre-shuffled weight, HBM-bound"),
    "bf16_256x8192x8192_preshuffled": Workload("bf16_256x8192x8192_preshuffled", 256, 8192, 8192, "bf16",
                                               "bf16", "bt_preshuffled", ("normal", 0.0, 1.0),
                                               ("normal", 0.0, 0.02), 1015,
                                               "batched decode / small prefill, pre-shuffled weight"),
    "bf16_1024x8192x8192": Workload("bf16_1024x8192x8192", 1024, 8192, 8192, "bf16", "bf16", "bt",
                                    ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), 1016,
                                    "prefill chunk: 128 output tiles"),
    "e4m3_1024x8192x8192": Workload("e4m3_1024x8192x8192", 1024, 8192, 8192, "e4m3", "bf16", "bt_preshuffled",
                                    ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1018,
                                    "prefill chunk in fp8, per-tensor scales amax/448, pre-shuffled weight"),
    "e4m3_8192": Workload("e4m3_8192", 8192, 8192, 8192, "e4m3", "bf16", "bt",
                          ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1005,
                          "per-tensor scales amax/448"),
    "e4m3_8192_preshuffled": Workload("e4m3_8192_preshuffled", 8192, 8192, 8192, "e4m3", "bf16", "bt_preshuffled",
                                      ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1005,
                                      "the same inputs as e4m3_8192, B pre-shuffled"),
    "mxfp8_8192": Workload("mxfp8_8192", 8192, 8192, 8192, "mxfp8", "bf16", "bt_preshuffled",
                           ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1006,
                           "MX block scales, e4m3 elements"),
    "mxfp4_32x8192x8192": Workload("mxfp4_32x8192x8192", 32, 8192, 8192, "mxfp4", "bf16", "bt_preshuffled",
                                   ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1019,
                                   "decode with an MXFP4 weight"),
    "mxfp4_8192": Workload("mxfp4_8192", 8192, 8192, 8192, "mxfp4", "bf16", "bt_preshuffled",
                           ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1007,
                           "MX block scales, e2m1 elements"),
    "bf16_4096_bn": Workload("bf16_4096_bn", 4096, 4096, 4096, "bf16", "bf16", "bn",
                             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1010,
                             "B stored K x N (C = A * B)"),
    "e4m3_8192_bn": Workload("e4m3_8192_bn", 8192, 8192, 8192, "e4m3", "bf16", "bn",
                             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1013,
                             "per-tensor scales amax/448, B stored K x N"),
    "bf16_4096_at": Workload("bf16_4096_at", 4096, 4096, 4096, "bf16", "bf16", "at",
                             ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1011,
                             "A stored K x M"),
    "bf16_4096_at_bn": Workload("bf16_4096_at_bn", 4096, 4096, 4096, "bf16", "bf16", "at_bn",
                                ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1012,
                                "A stored K x M, B stored K x N"),
    "i8_8192": Workload("i8_8192", 8192, 8192, 8192, "i8", "bf16", "bt_preshuffled",
                        ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1008,
                        "per-row / per-channel absmax scales"),
    "i8_8192_bt": Workload("i8_8192_bt", 8192, 8192, 8192, "i8", "bf16", "bt",
                           ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1021,
                           "per-row / per-channel absmax scales, B N x K"),
    "w4a8_32x8192x8192": Workload("w4a8_32x8192x8192", 32, 8192, 8192, "w4a8", "bf16", "bt_preshuffled",
                                  ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1017,
                                  "decode with an int4 weight: int8 A, packed int4 B"),
    "w4a8_256x8192x8192": Workload("w4a8_256x8192x8192", 256, 8192, 8192, "w4a8", "bf16", "bt_preshuffled",
                                   ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1020,
                                   "batched decode with an int4 weight"),
    "w4a8_8192": Workload("w4a8_8192", 8192, 8192, 8192, "w4a8", "bf16", "bt_preshuffled",
                          ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1009,
                          "int8 A, int4 B, per-row / per-channel absmax scales"),
}


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "int":
        return rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float32)
    if kind == "normal":
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(dist[2])
                + np.float32(dist[1])).astype(np.float32)
    if kind == "uniform":
        u = rng.random(size=shape, dtype=np.float32)          # [0, 1)
        return (u * np.float32(dist[2] - dist[1]) + np.float32(dist[1])).astype(np.float32)
    raise ValueError("unknown distribution %r" % (kind,))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (nearest-even) as uint16 bits, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def quantize_e4m3(x: np.ndarray):
    """Per-tensor e4m3fn quantisation: returns (uint8 bits, float32 scale)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    t = torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32)
    t = torch.clamp(t, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy(), float(s)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
MX_EMAX = {"mxfp8": 8, "mxfp4": 2}


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code, saturating at 6)."""
    a = np.minimum(np.abs(v.astype(np.float64)), 6.0)
    hi = np.clip(np.searchsorted(E2M1_GRID, a), 1, 7)
    lo = hi - 1
    d_lo, d_hi = a - E2M1_GRID[lo], E2M1_GRID[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(np.signbit(v) & (pick > 0), 8, 0)).astype(np.uint8)


def quantize_mx(x: np.ndarray, fmt: str):
    """MX quantisation of rows x K float32 data: (element bytes, E8M0 scales rows x K/32)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    blk = x.reshape(rows, K // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - MX_EMAX[fmt], -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    v = (blk / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K)
    if fmt == "mxfp8":
        t = torch.from_numpy(np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32)).to(torch.float8_e4m3fn)
        q = t.view(torch.uint8).numpy().copy()
    else:
        c = _e2m1_codes(v)
        q = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return q, (e + 127).astype(np.uint8)


def quantize_int_rows(x: np.ndarray, qmax: int):
    """Symmetric per-row absmax quantisation: (int8 values, float32 scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.size else np.zeros(x.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(qmax), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(x / s[:, None]), -qmax, qmax).astype(np.int8)
    return q, s


def pack_int4(q: np.ndarray) -> np.ndarray:
    """rows x K int4 values (int8 storage, -8..7) -> rows x K/2 bytes, the
    even element in the low nibble."""
    n = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def mx_int_inputs(M: int, N: int, K: int, fmt: str, seed: int):
    """Small MX inputs whose products and sums are exact in fp32: e4m3
    integers in [-4, 4] or any e2m1 code, with scales 2^-2 .. 2^2."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for rows in (M, N):
        if fmt == "mxfp8":
            import torch
            vals = rng.integers(-4, 5, size=(rows, K)).astype(np.float32)
            q = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        else:
            c = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
            q = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        out.append((q, rng.integers(125, 130, size=(rows, K // 32)).astype(np.uint8)))
    return Inputs(out[0][0], out[1][0], sa_blocks=out[0][1], sb_blocks=out[1][1])


@dataclass
class Inputs:
    A: np.ndarray          # raw bits, M x K (MXFP4: M x K/2 bytes)
    B: np.ndarray          # raw bits, N x K
    scale_a: float = 1.0
    scale_b: float = 1.0
    sa_blocks: np.ndarray | None = None   # MX: E8M0 scales, M x K/32
    sb_blocks: np.ndarray | None = None   # MX: E8M0 scales, N x K/32
    sa_rows: np.ndarray | None = None     # int8 / W4A8: float32 scale per row of A
    sb_cols: np.ndarray | None = None     # int8 / W4A8: float32 scale per row of B (column of C)


def make_inputs(w: Workload, M: int | None = None, N: int | None = None,
                K: int | None = None, seed: int | None = None) -> Inputs:
    """Inputs of workload ``w`` (optionally at another shape or seed)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    a = _draw(rng, w.dist_a, (M, K))
    b = _draw(rng, w.dist_b, (N, K))
    if w.dtype == "bf16":
        # drawn as M x K and N x K, then stored as the layout says
        if w.layout in ("bn", "at_bn"):
            b = np.ascontiguousarray(b.T)
        if w.layout in ("at", "at_bn"):
            a = np.ascontiguousarray(a.T)
        return Inputs(to_bf16_bits(a), to_bf16_bits(b))
    if w.dtype.startswith("mx"):
        qa, ea = quantize_mx(a, w.dtype)
        qb, eb = quantize_mx(b, w.dtype)
        return Inputs(qa, qb, sa_blocks=ea, sb_blocks=eb)
    if w.dtype in ("i8", "w4a8"):
        qa, sa = quantize_int_rows(a, 127)
        if w.dtype == "i8":
            qb, sb = quantize_int_rows(b, 127)
            qb = qb.view(np.uint8)
        else:
            qb, sb = quantize_int_rows(b, 7)
            qb = pack_int4(qb)
        return Inputs(qa.view(np.uint8), qb, sa_rows=sa, sb_cols=sb)
    qa, sa = quantize_e4m3(a)
    qb, sb = quantize_e4m3(b)
    if w.layout == "bn":
        qb = np.ascontiguousarray(qb.T)
    return Inputs(qa, qb, sa, sb)


def int_inputs(M: int, N: int, K: int, dtype: str, seed: int, lo: int = -4, hi: int = 4) -> Inputs:
    """Integer-valued inputs in [lo, hi] (exact in bf16 and e4m3 for |v| <= 16;
    for "i8" any range within int8, for "w4a8" B clipped to the int4 range)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype in ("i8", "w4a8"):
        a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.int8)
        if dtype == "i8":
            return Inputs(a.view(np.uint8), rng.integers(lo, hi + 1, size=(N, K)).astype(np.int8).view(np.uint8))
        b = rng.integers(max(lo, -8), min(hi, 7) + 1, size=(N, K)).astype(np.int8)
        return Inputs(a.view(np.uint8), pack_int4(b))
    a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    b = rng.integers(lo, hi + 1, size=(N, K)).astype(np.float32)
    if dtype == "bf16":
        return Inputs(to_bf16_bits(a), to_bf16_bits(b))
    import torch
    qa = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    qb = torch.from_numpy(b).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return Inputs(qa, qb, 1.0, 1.0)
