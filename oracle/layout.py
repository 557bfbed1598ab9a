"""Brute-force layout algebra and the B pre-shuffle permutation (TEST ORACLE).

A layout is a pair (shape, stride) of equally nested integer tuples; a
coordinate maps to the index sum(c_i * stride_i) over the flattened modes
(FlyDSL "Kernel Authoring" skill, section 2 "Layout System", "Coordinate
Mapping", worked example (8,16):(1,8): (3,5) -> 43 and back).

``idx2crd`` is the stride-aware inverse c_i = (idx // stride_i) % shape_i,
the reading under which the same section's ``(4,64):(64,1)`` layout turns a
thread index into (wave_id, lane_id); it is an inverse only for injective
layouts whose modes do not overlap.

The pre-shuffle (same page, section 6 "GEMM Pattern (Preshuffle)") stores B
(N x K, row-major) as the 5-mode array (N/16, Kbytes/64, 4, 16, 16) taken in
row-major order: n-block, 64-byte k-block, 16-byte k-quarter, row within the
n-block, byte.  Here it is written as a reshape + transpose of B's bytes.
"""
from __future__ import annotations

import itertools

import numpy as np


def flatten(t):
    """Flatten a nested int tuple into a list of ints."""
    if isinstance(t, (tuple, list)):
        out = []
        for x in t:
            out.extend(flatten(x))
        return out
    return [int(t)]


def size(shape) -> int:
    n = 1
    for s in flatten(shape):
        n *= s
    return n


def crd2idx(crd, shape, stride) -> int:
    """Index of a coordinate.  ``crd`` is either a tuple nested like ``shape``
    or a single integer, which is first split colexicographically over the
    flattened shape (mode 0 fastest)."""
    shp = flatten(shape)
    std = flatten(stride)
    if len(shp) != len(std):
        raise ValueError("shape/stride rank mismatch")
    if isinstance(crd, (tuple, list)):
        c = flatten(crd)
        if len(c) != len(shp):
            raise ValueError("coordinate rank mismatch")
    else:
        rest = int(crd)
        c = []
        for s in shp:
            c.append(rest % s)
            rest //= s
    return sum(ci * si for ci, si in zip(c, std))


def idx2crd(idx: int, shape, stride):
    shp = flatten(shape)
    std = flatten(stride)
    return tuple((int(idx) // d) % s for s, d in zip(shp, std))


def all_coords(shape):
    """Every coordinate of the flattened shape, mode 0 fastest."""
    shp = flatten(shape)
    for rev in itertools.product(*[range(s) for s in reversed(shp)]):
        yield tuple(reversed(rev))


def brute_force_table(shape, stride) -> np.ndarray:
    """Indices of every coordinate in colexicographic order."""
    return np.array([sum(c * d for c, d in zip(crd, flatten(stride)))
                     for crd in all_coords(shape)], dtype=np.int64)


def preshuffle_b_bytes(B: np.ndarray) -> np.ndarray:
    """Pre-shuffled byte image of B (N x K elements, row-major, 1 or 2 bytes
    each).  Requires N % 16 == 0 and (K * elem_bytes) % 64 == 0."""
    B = np.ascontiguousarray(B)
    N = B.shape[0]
    raw = B.view(np.uint8).reshape(N, -1)
    kb = raw.shape[1]
    if N % 16 or kb % 64:
        raise ValueError("preshuffle needs N % 16 == 0 and K*e % 64 == 0")
    five = raw.reshape(N // 16, 16, kb // 64, 4, 16)      # [nb][nr][kb][kq][byte]
    return np.ascontiguousarray(five.transpose(0, 2, 3, 1, 4)).reshape(-1)


def preshuffle_src_offset(n: int, kbyte: int, N: int, kbytes: int) -> int:
    """Byte offset in the pre-shuffled buffer of B's byte (n, kbyte)."""
    nb, nr = divmod(n, 16)
    kb, rem = divmod(kbyte, 64)
    kq, byte = divmod(rem, 16)
    return (((nb * (kbytes // 64) + kb) * 4 + kq) * 16 + nr) * 16 + byte


def bscale_image(S: np.ndarray, K: int) -> np.ndarray:
    """Block-scale image of MX scales S (R x K/32 E8M0 bytes): the bytes
    (ceil(R/64), G, 64, 4, 4), G = ceil(ceil(K/128)/4), where entry
    (quad, g, lane, b, s) is S[64 quad + 16 b + lane % 16][4 (4 g + s) + lane // 16],
    or 127 past the rows or the blocks.  Written out index by index."""
    S = np.asarray(S, np.uint8)
    R, kb = S.shape
    assert kb == K // 32
    groups = ((K + 127) // 128 + 3) // 4
    quads = (R + 63) // 64
    img = np.full((quads, groups, 64, 4, 4), 127, np.uint8)
    for quad in range(quads):
        for g in range(groups):
            for lane in range(64):
                for b in range(4):
                    row = 64 * quad + 16 * b + lane % 16
                    if row >= R:
                        continue
                    for s in range(4):
                        blk = 4 * (4 * g + s) + lane // 16
                        if blk < kb:
                            img[quad, g, lane, b, s] = S[row, blk]
    return img.reshape(-1)


def bscale_image_32(S: np.ndarray, K: int) -> np.ndarray:
    """Block-scale image, form 1 (the 32x32x64 MFMA's lane order): the same
    (ceil(R/64), G, 64, 4, 4) bytes, where entry (quad, g, lane, w, b) is
    S[64 quad + 32 (w // 2) + lane % 32][16 g + 2 (2 b + w % 2) + lane // 32],
    or 127 past the rows or the blocks.  Written out index by index."""
    S = np.asarray(S, np.uint8)
    R, kb = S.shape
    assert kb == K // 32
    groups = ((K + 127) // 128 + 3) // 4
    quads = (R + 63) // 64
    img = np.full((quads, groups, 64, 4, 4), 127, np.uint8)
    for quad in range(quads):
        for g in range(groups):
            for lane in range(64):
                for w in range(4):
                    row = 64 * quad + 32 * (w // 2) + lane % 32
                    if row >= R:
                        continue
                    for b in range(4):
                        blk = 16 * g + 2 * (2 * b + w % 2) + lane // 32
                        if blk < kb:
                            img[quad, g, lane, w, b] = S[row, blk]
    return img.reshape(-1)
