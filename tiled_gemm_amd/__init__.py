"""Python binding of ``libtgemm.so`` (the C ABI in ``include/tgemm.h``).

Argument marshalling only: every function below forwards to the C entry
point of the same name; all GEMM work runs in the library's HIP kernels.
Pointers are plain integers (``tensor.data_ptr()``), streams are HIP stream
handles (``torch.cuda.current_stream().cuda_stream``) or 0.

If the library has not been built, loading fails loudly: there is no
fallback path.  Build it with ``python -m tiled_gemm_amd.build`` or
``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtgemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_HIP = -3

GEMM_BF16_OUT_F32 = 0
GEMM_BF16_OUT_BF16 = 1
GEMM_E4M3_OUT_BF16 = 2
GEMM_MXFP8_OUT_BF16 = 3
GEMM_MXFP4_OUT_BF16 = 4
GEMM_I8_OUT_BF16 = 5           # int8 A and B, int32 sums
GEMM_W4A8_OUT_BF16 = 6         # int8 A, packed int4 B (two per byte, even element low)

GEMM_LAYOUT_BT = 0
GEMM_LAYOUT_BT_PRESHUFFLED = 1
GEMM_LAYOUT_BN = 2             # B stored K x N row-major: C = A * B
GEMM_LAYOUT_AT = 3             # A stored K x M row-major, B N x K
GEMM_LAYOUT_AT_BN = 4          # A stored K x M, B stored K x N

GEMM_EPI_NONE, GEMM_EPI_BIAS, GEMM_EPI_BIAS_RELU, GEMM_EPI_BIAS_SILU, GEMM_EPI_BIAS_GELU = range(5)
EPILOGUES = {"none": GEMM_EPI_NONE, "bias": GEMM_EPI_BIAS, "bias_relu": GEMM_EPI_BIAS_RELU,
             "bias_silu": GEMM_EPI_BIAS_SILU, "bias_gelu": GEMM_EPI_BIAS_GELU}

# gemm_kernel_choice (gemm_plan_create_opt)
GEMM_KERNEL_AUTO, GEMM_KERNEL_GENERIC_128, GEMM_KERNEL_GENERIC_256, GEMM_KERNEL_TILE256, GEMM_KERNEL_PIPE, \
    GEMM_KERNEL_PIPE4 = range(6)
KERNELS = {"auto": GEMM_KERNEL_AUTO, "generic128": GEMM_KERNEL_GENERIC_128, "generic256": GEMM_KERNEL_GENERIC_256,
           "tile256": GEMM_KERNEL_TILE256, "pipe": GEMM_KERNEL_PIPE, "pipe4": GEMM_KERNEL_PIPE4}

GEMM_MAX_RANK = 8
GEMM_VIEW_A, GEMM_VIEW_B, GEMM_VIEW_B_SHUF, GEMM_VIEW_B_SRC, GEMM_VIEW_C, GEMM_VIEW_LDS_A, GEMM_VIEW_TILE = range(7)

EXPORTS = (
    "gemm_plan_create", "gemm_plan_create_opt", "gemm_plan_destroy", "gemm_preshuffled_b_bytes", "gemm_preshuffle_b",
    "gemm_run", "gemm_run_ex", "gemm_bscale_image_bytes", "gemm_preshuffle_bscale", "gemm_run_mx",
    "gemm_last_error", "gemm_plan_query", "gemm_plan_layout", "gemm_layout_crd2idx",
    "gemm_layout_idx2crd", "gemm_lds_swizzle", "gemm_tile_of_workgroup", "gemm_workspace_bytes",
    "gemm_run_ws", "gemm_run_ws_noalloc",
)

GEMM_STATIC_WORKSPACE_BYTES = 64 << 20


class GemmError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__("%s failed (%d): %s" % (where, code, msg))
        self.code = code


class gemm_epilogue_args(ctypes.Structure):
    _fields_ = [("scale_a", ctypes.c_void_p), ("scale_b", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("scale_a_per_row", ctypes.c_int32), ("scale_b_per_col", ctypes.c_int32),
                ("epilogue", ctypes.c_int32)]


class gemm_plan_options(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("splits", ctypes.c_int32)]


class gemm_plan_info(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)] + [
        (f, ctypes.c_int32) for f in (
            "dtype", "layout", "elem_bytes", "out_bytes", "kernel", "tile_m", "tile_n",
            "tile_k_bytes", "threads", "lds_stages", "lds_bytes", "grid", "tiles_m", "tiles_n",
            "group_m", "split_k", "elem_bits", "b_elem_bits", "ws_splits", "ws_grid", "scale_form")]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def load() -> ctypes.CDLL:
    """Load the library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("tiled_gemm_amd: %s is not built; run `python -m tiled_gemm_amd.build` "
                           "(or __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    p64 = ctypes.POINTER(ctypes.c_int64)
    p32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "gemm_plan_create": (vp, [i64, i64, i64, c_int, c_int]),
        "gemm_plan_create_opt": (vp, [i64, i64, i64, c_int, c_int, ctypes.POINTER(gemm_plan_options)]),
        "gemm_plan_destroy": (None, [vp]),
        "gemm_preshuffled_b_bytes": (ctypes.c_size_t, [vp]),
        "gemm_preshuffle_b": (c_int, [vp, vp, vp, vp]),
        "gemm_run": (c_int, [vp, vp, vp, vp, vp, vp]),
        "gemm_run_ex": (c_int, [vp, vp, vp, vp, ctypes.POINTER(gemm_epilogue_args), vp]),
        "gemm_bscale_image_bytes": (ctypes.c_size_t, [vp, c_int]),
        "gemm_preshuffle_bscale": (c_int, [vp, c_int, vp, vp, vp]),
        "gemm_run_mx": (c_int, [vp, vp, vp, vp, vp, vp, ctypes.POINTER(gemm_epilogue_args), vp]),
        "gemm_workspace_bytes": (ctypes.c_size_t, [vp]),
        "gemm_run_ws": (c_int, [vp, vp, vp, vp, ctypes.POINTER(gemm_epilogue_args), vp, ctypes.c_size_t, vp]),
        "gemm_run_ws_noalloc": (c_int, [vp, vp, vp, vp, ctypes.POINTER(gemm_epilogue_args), vp]),
        "gemm_last_error": (ctypes.c_char_p, []),
        "gemm_plan_query": (c_int, [vp, ctypes.POINTER(gemm_plan_info)]),
        "gemm_plan_layout": (c_int, [vp, c_int, p32, p64, p64]),
        "gemm_layout_crd2idx": (i64, [i32, p64, p64, p64]),
        "gemm_layout_idx2crd": (c_int, [i32, p64, p64, i64, p64]),
        "gemm_lds_swizzle": (i32, [i32, i32, i32]),
        "gemm_tile_of_workgroup": (c_int, [vp, i32, p32, p32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def gemm_last_error() -> str:
    return load().gemm_last_error().decode()


def _check(rc: int, where: str) -> int:
    if rc != GEMM_OK:
        raise GemmError(rc, where, gemm_last_error())
    return rc


def _arr64(vals):
    vals = list(vals)
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


# ---------------------------------------------------------------- entry points

def gemm_plan_create(M: int, N: int, K: int, dtype: int, layout: int) -> int:
    h = load().gemm_plan_create(M, N, K, dtype, layout)
    if not h:
        raise GemmError(-1, "gemm_plan_create", gemm_last_error())
    return h


def gemm_plan_create_opt(M: int, N: int, K: int, dtype: int, layout: int, kernel: int = GEMM_KERNEL_AUTO,
                         splits: int = 0) -> int:
    opt = gemm_plan_options(kernel, splits)
    h = load().gemm_plan_create_opt(M, N, K, dtype, layout, ctypes.byref(opt))
    if not h:
        raise GemmError(-1, "gemm_plan_create_opt", gemm_last_error())
    return h


def gemm_plan_destroy(plan: int) -> None:
    load().gemm_plan_destroy(plan)


def gemm_preshuffled_b_bytes(plan: int) -> int:
    return int(load().gemm_preshuffled_b_bytes(plan))


def gemm_preshuffle_b(plan: int, B: int, B_shuf: int, stream: int = 0) -> None:
    _check(load().gemm_preshuffle_b(plan, B, B_shuf, stream), "gemm_preshuffle_b")


def gemm_run(plan: int, A: int, B: int, C: int, scale: int | None = None, stream: int = 0) -> None:
    _check(load().gemm_run(plan, A, B, C, scale or None, stream), "gemm_run")


def gemm_run_ex(plan: int, A: int, B: int, C: int, scale_a: int | None = None, scale_a_per_row: bool = False,
                scale_b: int | None = None, scale_b_per_col: bool = False, bias: int | None = None,
                epilogue: int = GEMM_EPI_NONE, stream: int = 0) -> None:
    epi = gemm_epilogue_args(scale_a or None, scale_b or None, bias or None, int(scale_a_per_row),
                             int(scale_b_per_col), epilogue)
    _check(load().gemm_run_ex(plan, A, B, C, ctypes.byref(epi), stream), "gemm_run_ex")


def gemm_workspace_bytes(plan: int) -> int:
    return int(load().gemm_workspace_bytes(plan))


def gemm_run_ws(plan: int, A: int, B: int, C: int, workspace: int | None, workspace_bytes: int,
                scale_a: int | None = None, scale_a_per_row: bool = False, scale_b: int | None = None,
                scale_b_per_col: bool = False, bias: int | None = None, epilogue: int = GEMM_EPI_NONE,
                stream: int = 0) -> None:
    epi = gemm_epilogue_args(scale_a or None, scale_b or None, bias or None, int(scale_a_per_row),
                             int(scale_b_per_col), epilogue)
    _check(load().gemm_run_ws(plan, A, B, C, ctypes.byref(epi), workspace or None, workspace_bytes, stream),
           "gemm_run_ws")


def gemm_run_ws_noalloc(plan: int, A: int, B: int, C: int, scale_a: int | None = None,
                        scale_a_per_row: bool = False, scale_b: int | None = None, scale_b_per_col: bool = False,
                        bias: int | None = None, epilogue: int = GEMM_EPI_NONE, stream: int = 0) -> None:
    epi = gemm_epilogue_args(scale_a or None, scale_b or None, bias or None, int(scale_a_per_row),
                             int(scale_b_per_col), epilogue)
    _check(load().gemm_run_ws_noalloc(plan, A, B, C, ctypes.byref(epi), stream), "gemm_run_ws_noalloc")


def gemm_bscale_image_bytes(plan: int, operand: int) -> int:
    return int(load().gemm_bscale_image_bytes(plan, operand))


def gemm_preshuffle_bscale(plan: int, operand: int, scales: int, image: int, stream: int = 0) -> None:
    _check(load().gemm_preshuffle_bscale(plan, operand, scales, image, stream), "gemm_preshuffle_bscale")


def gemm_run_mx(plan: int, A: int, A_bscale: int, B: int, B_bscale: int, C: int, scale_a: int | None = None,
                scale_a_per_row: bool = False, scale_b: int | None = None, scale_b_per_col: bool = False,
                bias: int | None = None, epilogue: int = GEMM_EPI_NONE, stream: int = 0) -> None:
    epi = gemm_epilogue_args(scale_a or None, scale_b or None, bias or None, int(scale_a_per_row),
                             int(scale_b_per_col), epilogue)
    _check(load().gemm_run_mx(plan, A, A_bscale, B, B_bscale, C, ctypes.byref(epi), stream), "gemm_run_mx")


def gemm_plan_query(plan: int) -> dict:
    info = gemm_plan_info()
    _check(load().gemm_plan_query(plan, ctypes.byref(info)), "gemm_plan_query")
    return info.as_dict()


def gemm_plan_layout(plan: int, view: int):
    rank = ctypes.c_int32(0)
    shape = (ctypes.c_int64 * GEMM_MAX_RANK)()
    stride = (ctypes.c_int64 * GEMM_MAX_RANK)()
    _check(load().gemm_plan_layout(plan, view, ctypes.byref(rank), shape, stride), "gemm_plan_layout")
    r = rank.value
    return tuple(shape[:r]), tuple(stride[:r])


def gemm_layout_crd2idx(shape, stride, crd) -> int:
    v = load().gemm_layout_crd2idx(len(shape), _arr64(shape), _arr64(stride), _arr64(crd))
    if v < 0:
        raise GemmError(GEMM_ERR_INVALID_ARG, "gemm_layout_crd2idx", gemm_last_error())
    return int(v)


def gemm_layout_idx2crd(shape, stride, idx: int):
    out = (ctypes.c_int64 * GEMM_MAX_RANK)()
    _check(load().gemm_layout_idx2crd(len(shape), _arr64(shape), _arr64(stride), idx, out),
           "gemm_layout_idx2crd")
    return tuple(out[:len(shape)])


def gemm_lds_swizzle(row: int, chunk: int, chunks_per_row: int = 8) -> int:
    v = load().gemm_lds_swizzle(row, chunk, chunks_per_row)
    if v < 0:
        raise GemmError(GEMM_ERR_INVALID_ARG, "gemm_lds_swizzle", gemm_last_error())
    return int(v)


def gemm_tile_of_workgroup(plan: int, wg: int):
    tm, tn = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().gemm_tile_of_workgroup(plan, wg, ctypes.byref(tm), ctypes.byref(tn)),
           "gemm_tile_of_workgroup")
    return tm.value, tn.value


# ---------------------------------------------------------------- conveniences

DTYPES = {"bf16_f32": GEMM_BF16_OUT_F32, "bf16": GEMM_BF16_OUT_BF16, "e4m3": GEMM_E4M3_OUT_BF16,
          "mxfp8": GEMM_MXFP8_OUT_BF16, "mxfp4": GEMM_MXFP4_OUT_BF16, "i8": GEMM_I8_OUT_BF16,
          "w4a8": GEMM_W4A8_OUT_BF16}
LAYOUTS = {"bt": GEMM_LAYOUT_BT, "bt_preshuffled": GEMM_LAYOUT_BT_PRESHUFFLED, "bn": GEMM_LAYOUT_BN,
           "at": GEMM_LAYOUT_AT, "at_bn": GEMM_LAYOUT_AT_BN}


class Plan:
    """Owns one plan handle; ``with Plan(...) as p:`` destroys it on exit.
    ``kernel`` (a gemm_kernel_choice) and ``splits`` go to
    gemm_plan_create_opt; the defaults are gemm_plan_create."""

    def __init__(self, M: int, N: int, K: int, dtype: int, layout: int, kernel: int = GEMM_KERNEL_AUTO,
                 splits: int = 0):
        self.handle = 0                      # set before create, which may raise
        if kernel == GEMM_KERNEL_AUTO and splits == 0:
            self.handle = gemm_plan_create(M, N, K, dtype, layout)
        else:
            self.handle = gemm_plan_create_opt(M, N, K, dtype, layout, kernel, splits)

    def close(self):
        h, self.handle = self.handle, 0
        # At interpreter exit the module's globals may already be cleared.
        destroy = globals().get("gemm_plan_destroy")
        if h and destroy is not None:
            destroy(h)

    __del__ = close

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def info(self) -> dict:
        return gemm_plan_query(self.handle)

    def preshuffle_b(self, B: int, B_shuf: int, stream: int = 0) -> None:
        gemm_preshuffle_b(self.handle, B, B_shuf, stream)

    def run(self, A: int, B: int, C: int, scale: int | None = None, stream: int = 0) -> None:
        gemm_run(self.handle, A, B, C, scale, stream)

    def bscale_image_bytes(self, operand: int) -> int:
        return gemm_bscale_image_bytes(self.handle, operand)

    def preshuffle_bscale(self, operand: int, scales: int, image: int, stream: int = 0) -> None:
        gemm_preshuffle_bscale(self.handle, operand, scales, image, stream)

    def run_mx(self, A: int, A_bscale: int, B: int, B_bscale: int, C: int, stream: int = 0, **epi) -> None:
        gemm_run_mx(self.handle, A, A_bscale, B, B_bscale, C, stream=stream, **epi)

    def run_ex(self, A: int, B: int, C: int, stream: int = 0, **epi) -> None:
        """gemm_run_ex; keyword arguments as for the module-level gemm_run_ex."""
        gemm_run_ex(self.handle, A, B, C, stream=stream, **epi)

    def workspace_bytes(self) -> int:
        return gemm_workspace_bytes(self.handle)

    def run_ws(self, A: int, B: int, C: int, workspace: int | None, workspace_bytes: int, stream: int = 0,
               **epi) -> None:
        """gemm_run_ws; keyword arguments as for the module-level gemm_run_ex."""
        gemm_run_ws(self.handle, A, B, C, workspace, workspace_bytes, stream=stream, **epi)

    def run_ws_noalloc(self, A: int, B: int, C: int, stream: int = 0, **epi) -> None:
        """gemm_run_ws_noalloc; keyword arguments as for the module-level gemm_run_ex."""
        gemm_run_ws_noalloc(self.handle, A, B, C, stream=stream, **epi)
