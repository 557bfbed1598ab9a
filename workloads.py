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

A is M x K, B is N x K (K contiguous in both), C is M x N.
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
    dtype: str          # "bf16" or "e4m3" (element type of A and B)
    out: str            # "f32" or "bf16"
    layout: str         # "bt" (B as N x K) or "bt_preshuffled"
    dist_a: tuple
    dist_b: tuple
    seed: int
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 1

    @property
    def out_bytes(self) -> int:
        return 4 if self.out == "f32" else 2

    @property
    def min_bytes(self) -> int:
        """Each operand read once and C written once."""
        return (self.M * self.K + self.N * self.K) * self.elem_bytes + self.M * self.N * self.out_bytes


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
    "e4m3_8192": Workload("e4m3_8192", 8192, 8192, 8192, "e4m3", "bf16", "bt",
                          ("normal", 0.0, 1.0), ("normal", 0.0, 1.0), 1005,
                          "per-tensor scales amax/448"),
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


@dataclass
class Inputs:
    A: np.ndarray          # raw bits, M x K
    B: np.ndarray          # raw bits, N x K
    scale_a: float = 1.0
    scale_b: float = 1.0


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
        return Inputs(to_bf16_bits(a), to_bf16_bits(b))
    qa, sa = quantize_e4m3(a)
    qb, sb = quantize_e4m3(b)
    return Inputs(qa, qb, sa, sb)


def int_inputs(M: int, N: int, K: int, dtype: str, seed: int, lo: int = -4, hi: int = 4) -> Inputs:
    """Integer-valued inputs in [lo, hi] (exact in bf16 and e4m3 for |v| <= 16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    b = rng.integers(lo, hi + 1, size=(N, K)).astype(np.float32)
    if dtype == "bf16":
        return Inputs(to_bf16_bits(a), to_bf16_bits(b))
    import torch
    qa = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    qb = torch.from_numpy(b).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return Inputs(qa, qb, 1.0, 1.0)
