"""CPU oracle for the tiled GEMM C = A * B^T -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
under ``tiled_gemm_amd/`` and never imports it.

Contents
--------
* ``gemm_bt`` / ``gemm_bt_entries`` -- the fp64 triple loop in ``oracle.c``
  (plain i-j-k, sequential k, sigma = s_a * s_b for fp8), built with gcc.
* ``epilogue`` -- the fused epilogue (scale vectors, bias, ReLU / SiLU /
  GELU) applied in fp64 to the exact GEMM result.
* ``gemm_bt_mx`` / ``gemm_bt_mx_entries`` -- the same loop for MX
  block-scaled operands (MXFP8: e4m3 elements, MXFP4: e2m1 elements, one
  E8M0 scale per 32 elements along K).
* ``gemm_ab`` / ``gemm_ab_entries`` -- C = A * B with B stored K x N (the
  naive template's layout): b(n, k) is B[k][n], i.e. the same sum with the
  stored B read column-wise.
* ``gemm_at`` / ``gemm_at_entries`` -- the same sum with A stored K x M:
  a(m, k) is A[k][m] (and, with ``b_kn``, B stored K x N as well).
* ``gemm_bt_int`` / ``gemm_bt_int_entries`` -- exact integer sums (int64)
  for an int8 A and an int8 or packed int4 B (W4A8).
* ``round_bf16`` -- the oracle's own round-to-nearest-even to bf16.
* ``bf16_value`` / ``e4m3fn_value`` -- element decoders from the format
  definitions.
* ``layout`` -- brute-force layout algebra (``crd2idx``/``idx2crd``) and the
  B pre-shuffle permutation written as a reshape/transpose.

Every function's pins are in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
E4M3FN = 1
MXFP8 = 2
MXFP4 = 3

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_bf16_value.restype = dbl
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3fn_value.restype = dbl
    lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
    lib.oracle_gemm_bt.restype = None
    lib.oracle_gemm_bt.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, dbl, vp, vp]
    lib.oracle_gemm_bt_entries.restype = None
    lib.oracle_gemm_bt_entries.argtypes = [i64, ctypes.c_int, vp, vp, dbl, i64, vp, vp, vp, vp]
    lib.oracle_e2m1_value.restype = dbl
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = dbl
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_gemm_bt_mx.restype = None
    lib.oracle_gemm_bt_mx.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    lib.oracle_gemm_bt_mx_entries.restype = None
    lib.oracle_gemm_bt_mx_entries.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.oracle_int8_value.restype = ctypes.c_int
    lib.oracle_int8_value.argtypes = [ctypes.c_uint8]
    lib.oracle_int4_value.restype = ctypes.c_int
    lib.oracle_int4_value.argtypes = [ctypes.c_uint8]
    lib.oracle_gemm_bt_int.restype = None
    lib.oracle_gemm_bt_int.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, vp, vp]
    lib.oracle_gemm_bt_int_entries.restype = None
    lib.oracle_gemm_bt_int_entries.argtypes = [i64, ctypes.c_int, vp, vp, i64, vp, vp, vp, vp]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [dbl]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_bf16_array.argtypes = [i64, vp, vp]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle uses (``OMP_NUM_THREADS`` or all cores)."""
    return int(_load().oracle_threads())


def _kind(dtype: str) -> int:
    if dtype == "bf16":
        return BF16
    if dtype == "e4m3":
        return E4M3FN
    raise ValueError("oracle: unknown element type %r" % (dtype,))


def _operand(x: np.ndarray, dtype: str) -> np.ndarray:
    want = np.uint16 if dtype == "bf16" else np.uint8
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError("oracle: %s operand must hold raw %s bits" % (dtype, want.__name__))
    return x


def sigma_of(scale_a: float = 1.0, scale_b: float = 1.0) -> float:
    """sigma = s_a * s_b formed in fp64 from the two fp32 scales."""
    return float(np.float64(np.float32(scale_a)) * np.float64(np.float32(scale_b)))


def gemm_bt(A: np.ndarray, B: np.ndarray, dtype: str = "bf16", sigma: float = 1.0,
            want_s: bool = True):
    """Full C_ref (M x N, fp64) and S, for A (M x K) and B (N x K) raw bits."""
    A = _operand(A, dtype)
    B = _operand(B, dtype)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("oracle: K mismatch")
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64) if want_s else None
    _load().oracle_gemm_bt(M, N, K, _kind(dtype), A.ctypes.data, B.ctypes.data, float(sigma),
                           C.ctypes.data, S.ctypes.data if want_s else None)
    return C, S


def gemm_bt_entries(A: np.ndarray, B: np.ndarray, rows, cols, dtype: str = "bf16",
                    sigma: float = 1.0):
    """C_ref and S at the (rows[t], cols[t]) entries only."""
    A = _operand(A, dtype)
    B = _operand(B, dtype)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("oracle: rows/cols shape mismatch")
    K = A.shape[1]
    if B.shape[1] != K:
        raise ValueError("oracle: K mismatch")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0]
                      or cols.min() < 0 or cols.max() >= B.shape[0]):
        raise IndexError("oracle: entry out of range")
    C = np.empty(rows.shape, np.float64)
    S = np.empty(rows.shape, np.float64)
    _load().oracle_gemm_bt_entries(K, _kind(dtype), A.ctypes.data, B.ctypes.data, float(sigma),
                                   rows.size, rows.ctypes.data, cols.ctypes.data,
                                   C.ctypes.data, S.ctypes.data)
    return C, S


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(int(bits)))


def e4m3fn_value(bits: int) -> float:
    return float(_load().oracle_e4m3fn_value(int(bits)))


from . import layout  # noqa: E402,F401  (brute-force layout algebra)


# ------------------------------------------------------------------ epilogue

ACTIVATIONS = ("none", "bias", "bias_relu", "bias_silu", "bias_gelu")


def _logistic(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z), evaluated without overflow on either side."""
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def _std_normal_cdf(z: np.ndarray) -> np.ndarray:
    """Phi(z) = (1 + erf(z / sqrt 2)) / 2, with math.erf per element (fp64)."""
    import math
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0)))


def epilogue(acc: np.ndarray, scale_a=None, scale_b=None, bias=None, kind: str = "none") -> np.ndarray:
    """The fused epilogue on an exact GEMM result ``acc`` (M x N, fp64).

    FlyDSL "Kernel authoring guide", section 11 "Complete example: Preshuffle
    GEMM": the GEMM takes scale_a, scale_b and bias tensors and an epilogue of
    none / bias / bias_relu / bias_silu / bias_gelu; FlyDSL "Kernel Authoring"
    skill, section 3, applies the scales as (acc * scale_a) * scale_b.  The
    reading taken where the pages stop (shapes and activation formulas):

        z = (acc * sa[m]) * sb[n] + bias[n]
        relu: z if z > 0 else +0;   silu: z * logistic(z);
        gelu: z * Phi(z)  (the definition, not the tanh approximation)

    ``scale_a``: None, a scalar, or M values (per row); ``scale_b``: None, a
    scalar, or N values (per column); ``bias``: N values, used by every kind
    except "none".  Everything is fp64; no rounding to the output type.
    """
    if kind not in ACTIVATIONS:
        raise ValueError("unknown epilogue %r" % kind)
    acc = np.asarray(acc, dtype=np.float64)
    M, N = acc.shape
    sa = None if scale_a is None else np.broadcast_to(
        np.asarray(scale_a, np.float64).reshape(-1, 1) if np.ndim(scale_a) else np.float64(scale_a), (M, N))
    sb = None if scale_b is None else np.broadcast_to(
        np.asarray(scale_b, np.float64).reshape(1, -1) if np.ndim(scale_b) else np.float64(scale_b), (M, N))
    bz = None if kind == "none" else np.broadcast_to(np.asarray(bias, np.float64).reshape(1, -1), (M, N))
    return epilogue_entries(acc, sa, sb, bz, kind)


def epilogue_entries(acc, sa=None, sb=None, bias=None, kind: str = "none") -> np.ndarray:
    """The same epilogue element by element: z = (acc * sa) * sb + bias, then
    the activation; every argument an array of the same shape (or None for
    sa = 1, sb = 1, and no bias with kind "none")."""
    if kind not in ACTIVATIONS:
        raise ValueError("unknown epilogue %r" % kind)
    z = np.array(acc, dtype=np.float64, copy=True)
    if sa is not None:
        z = z * np.asarray(sa, np.float64)
    if sb is not None:
        z = z * np.asarray(sb, np.float64)
    if kind == "none":
        return z
    z = z + np.asarray(bias, np.float64)
    if kind == "bias_relu":
        return np.where(z > 0, z, 0.0)
    if kind == "bias_silu":
        return z * _logistic(z)
    if kind == "bias_gelu":
        return z * _std_normal_cdf(z)
    return z


# Largest slope of each activation (max over z of |d act / dz|), used by the
# tests to carry the GEMM's error bound through the activation: 1 for the
# identity and ReLU; SiLU peaks at 1.0998 (z ~ 2.40), GELU at 1.1290 (z ~ 1.41).
ACT_LIPSCHITZ = {"none": 1.0, "bias": 1.0, "bias_relu": 1.0, "bias_silu": 1.1, "bias_gelu": 1.13}


# ------------------------------------------------------------------ MX operands

def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code) & 0xF))


def e8m0_value(bits: int) -> float:
    return float(_load().oracle_e8m0_value(int(bits) & 0xFF))


def _mx(fmt: str):
    if fmt == "mxfp8":
        return MXFP8
    if fmt == "mxfp4":
        return MXFP4
    raise ValueError("oracle: unknown MX format %r" % (fmt,))


def _mx_operand(x, s, K: int, fmt: str):
    x = np.ascontiguousarray(x, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows = x.shape[0]
    if K % 32 or x.shape[1] != (K if fmt == "mxfp8" else K // 2) or s.shape != (rows, K // 32):
        raise ValueError("oracle: MX operand shape (rows x K%s, scales rows x K/32)" %
                         ("" if fmt == "mxfp8" else "/2 bytes"))
    return x, s


def gemm_bt_mx(A, SA, B, SB, K: int, fmt: str = "mxfp8", want_s: bool = True):
    """Full C_ref (fp64) and S for MX operands: A (M x K elements), B (N x K),
    element bytes row-major (MXFP4: two per byte, even element in the low
    nibble), scales SA (M x K/32), SB (N x K/32) E8M0 bytes."""
    A, SA = _mx_operand(A, SA, K, fmt)
    B, SB = _mx_operand(B, SB, K, fmt)
    M, N = A.shape[0], B.shape[0]
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64) if want_s else None
    _load().oracle_gemm_bt_mx(M, N, K, _mx(fmt), A.ctypes.data, SA.ctypes.data, B.ctypes.data, SB.ctypes.data,
                              C.ctypes.data, S.ctypes.data if want_s else None)
    return C, S


def gemm_bt_mx_entries(A, SA, B, SB, K: int, rows, cols, fmt: str = "mxfp8"):
    """C_ref and S of MX operands at the (rows[t], cols[t]) entries only."""
    A, SA = _mx_operand(A, SA, K, fmt)
    B, SB = _mx_operand(B, SB, K, fmt)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0 or cols.max() >= B.shape[0]):
        raise IndexError("oracle: entry out of range")
    C = np.empty(rows.shape, np.float64)
    S = np.empty(rows.shape, np.float64)
    _load().oracle_gemm_bt_mx_entries(K, _mx(fmt), A.ctypes.data, SA.ctypes.data, B.ctypes.data, SB.ctypes.data,
                                      rows.size, rows.ctypes.data, cols.ctypes.data, C.ctypes.data, S.ctypes.data)
    return C, S


# ---------------------------------------------------------------------------
# Integer operands: int8 A, int8 or packed int4 B (W4A8).
# ---------------------------------------------------------------------------
INT_B_BITS = {"i8": 8, "w4a8": 4}


def int8_value(bits: int) -> int:
    return int(_load().oracle_int8_value(int(bits) & 0xFF))


def int4_value(nibble: int) -> int:
    return int(_load().oracle_int4_value(int(nibble) & 0xF))


def _int_operands(A, B, K: int, fmt: str):
    if fmt not in INT_B_BITS:
        raise ValueError("oracle: unknown integer format %r" % (fmt,))
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    bb = INT_B_BITS[fmt]
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != K or B.shape[1] * 8 != K * bb:
        raise ValueError("oracle: integer operands are M x K bytes and N x K*%d/8 bytes" % bb)
    return A, B, bb


def gemm_bt_int(A, B, K: int, fmt: str = "i8", want_s: bool = True):
    """Exact acc = A * B^T and S = sum |a b| (as float64, exact below 2^53)
    for an int8 A (M x K) and B int8 (N x K, fmt "i8") or packed int4
    (N x K/2 bytes, fmt "w4a8")."""
    A, B, bb = _int_operands(A, B, K, fmt)
    M, N = A.shape[0], B.shape[0]
    C = np.empty((M, N), np.int64)
    S = np.empty((M, N), np.int64) if want_s else None
    _load().oracle_gemm_bt_int(M, N, K, bb, A.ctypes.data, B.ctypes.data, C.ctypes.data,
                               S.ctypes.data if want_s else None)
    return C.astype(np.float64), (S.astype(np.float64) if want_s else None)


def gemm_bt_int_entries(A, B, K: int, rows, cols, fmt: str = "i8"):
    """acc and S of the integer product at the (rows[t], cols[t]) entries."""
    A, B, bb = _int_operands(A, B, K, fmt)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0 or cols.max() >= B.shape[0]):
        raise IndexError("oracle: entry out of range")
    C = np.empty(rows.shape, np.int64)
    S = np.empty(rows.shape, np.int64)
    _load().oracle_gemm_bt_int_entries(K, bb, A.ctypes.data, B.ctypes.data, rows.size, rows.ctypes.data,
                                       cols.ctypes.data, C.ctypes.data, S.ctypes.data)
    return C.astype(np.float64), S.astype(np.float64)


# ---------------------------------------------------------------------------
# B stored K x N (C = A * B)
# ---------------------------------------------------------------------------
def gemm_ab(A: np.ndarray, B_kn: np.ndarray, dtype: str = "bf16", sigma: float = 1.0, want_s: bool = True):
    """C_ref[m][n] = sigma * sum_k a(m,k) * B_kn[k][n] for B stored K x N:
    the element B_kn[k][n] is b(n,k) of the N x K form, so this is gemm_bt on
    the transposed copy."""
    B_kn = _operand(B_kn, dtype)
    return gemm_bt(A, np.ascontiguousarray(B_kn.T), dtype=dtype, sigma=sigma, want_s=want_s)


def gemm_ab_entries(A: np.ndarray, B_kn: np.ndarray, rows, cols, dtype: str = "bf16", sigma: float = 1.0):
    """gemm_ab at the (rows[t], cols[t]) entries only."""
    B_kn = _operand(B_kn, dtype)
    return gemm_bt_entries(A, np.ascontiguousarray(B_kn.T), rows, cols, dtype=dtype, sigma=sigma)


def gemm_at(A_km: np.ndarray, B: np.ndarray, dtype: str = "bf16", sigma: float = 1.0, want_s: bool = True,
            b_kn: bool = False):
    """C_ref[m][n] = sigma * sum_k A_km[k][m] * b(n,k) for A stored K x M: the
    element A_km[k][m] is a(m,k) of the M x K form; B is N x K, or K x N with
    b_kn (b(n,k) = B[k][n]).  gemm_bt on the transposed copies."""
    A = np.ascontiguousarray(_operand(A_km, dtype).T)
    Bt = np.ascontiguousarray(_operand(B, dtype).T) if b_kn else B
    return gemm_bt(A, Bt, dtype=dtype, sigma=sigma, want_s=want_s)


def gemm_at_entries(A_km: np.ndarray, B: np.ndarray, rows, cols, dtype: str = "bf16", sigma: float = 1.0,
                    b_kn: bool = False):
    """gemm_at at the (rows[t], cols[t]) entries only."""
    A = np.ascontiguousarray(_operand(A_km, dtype).T)
    Bt = np.ascontiguousarray(_operand(B, dtype).T) if b_kn else B
    return gemm_bt_entries(A, Bt, rows, cols, dtype=dtype, sigma=sigma)
