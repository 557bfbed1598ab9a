"""Helpers for the GPU parity tests: device upload, one GEMM through the C
ABI, decoding of C, and the element-wise acceptance bound.

Acceptance (per element):  |C - C_ref| <= 4e-6 * S + rho * |C_ref|, with
S = |sigma| * sum_k |a_ik * b_jk| from the oracle, rho = 2^-8 for bf16 inputs
and 2^-3 for fp8 inputs; NaN or Inf anywhere fails.  Integer-valued inputs
whose partial sums are exact in fp32 must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import tiled_gemm_amd as tg

# MX: products of the decoded elements are exact in fp32, so only the fp32
# accumulation (the S term) and the output rounding (2^-8) remain.
# Integer operands: the sums are exact, so only the output rounding remains.
RHO = {"bf16": 2.0 ** -8, "e4m3": 2.0 ** -3, "mxfp8": 2.0 ** -8, "mxfp4": 2.0 ** -8, "i8": 2.0 ** -8,
       "w4a8": 2.0 ** -8}
ABS_COEF = 4e-6

# Kernel choice and split count for the plans run_gemm creates (see
# gemm_plan_create_opt); tests set them through the ``plan_opts`` fixture,
# which restores the planner's own choice afterwards.
PLAN_OPTS = {"kernel": 0, "splits": 0}

# Short names of the kernel families (gemm_kernel_choice): "generic128" /
# "generic256" the generic tiled kernel, "tile256" the planner's 256 x 256
# kernel at any size, "pipe" the 8-wave software-pipelined kernel with B in
# registers, "pipe4" its 4-wave AGPR form (MX: the 16x16x128 kernel).

DTYPE_CODE = {("bf16", "f32"): tg.GEMM_BF16_OUT_F32, ("bf16", "bf16"): tg.GEMM_BF16_OUT_BF16,
              ("e4m3", "bf16"): tg.GEMM_E4M3_OUT_BF16, ("mxfp8", "bf16"): tg.GEMM_MXFP8_OUT_BF16,
              ("mxfp4", "bf16"): tg.GEMM_MXFP4_OUT_BF16, ("i8", "bf16"): tg.GEMM_I8_OUT_BF16,
              ("w4a8", "bf16"): tg.GEMM_W4A8_OUT_BF16}


def to_dev(bits: np.ndarray) -> torch.Tensor:
    bits = np.ascontiguousarray(bits)
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).cuda()
    return torch.from_numpy(bits).cuda()


def _dev_f32(x):
    return torch.tensor(np.atleast_1d(np.asarray(x, np.float32)), dtype=torch.float32, device="cuda")


def run_gemm(A_bits, B_bits, M, N, K, dtype="bf16", out="bf16", layout="bt",
             scale=(1.0, 1.0), use_scale=True, stream=None, plan=None, return_plan_info=False, epi=None,
             sa_blocks=None, sb_blocks=None, workspace=None):
    """One C = A * B^T through gemm_plan_create / [gemm_preshuffle_b] /
    gemm_run, or gemm_run_ex when ``epi`` is given: a dict with optional
    scale_a (scalar or M values), scale_b (scalar or N values), bias (N
    values) and kind (a name in tg.EPILOGUES).  MX dtypes take the E8M0 block
    scales sa_blocks (M x K/32) and sb_blocks (N x K/32) and run through
    gemm_preshuffle_bscale + gemm_run_mx.  Returns the raw bits of C as a
    numpy array (M x N).  ``workspace`` runs gemm_run_ws: True gives it
    gemm_workspace_bytes(plan) bytes, an int that many (0: a NULL workspace);
    per-tensor ``scale`` then goes in as the epilogue's two scalars."""
    code = DTYPE_CODE[(dtype, out)]
    lay = tg.LAYOUTS[layout]
    own = plan is None
    if own:
        plan = tg.Plan(M, N, K, code, lay, **PLAN_OPTS)
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    ob = 4 if out == "f32" else 2
    A = to_dev(A_bits) if A_bits.size else torch.empty(16, dtype=torch.uint8, device="cuda")
    B = to_dev(B_bits) if B_bits.size else torch.empty(16, dtype=torch.uint8, device="cuda")
    Bx = B
    if layout == "bt_preshuffled" and B_bits.size:
        Bx = torch.empty(tg.gemm_preshuffled_b_bytes(plan.handle), dtype=torch.uint8, device="cuda")
        plan.preshuffle_b(B.data_ptr(), Bx.data_ptr(), s)
    C = torch.full((max(1, M * N * ob),), 0x5A, dtype=torch.uint8, device="cuda")
    if dtype.startswith("mx"):
        e = epi or {}
        keep = {k: _dev_f32(e[k]) for k in ("scale_a", "scale_b", "bias") if e.get(k) is not None}
        imgs = []
        for operand, blocks in ((0, sa_blocks), (1, sb_blocks)):
            src = torch.from_numpy(np.ascontiguousarray(blocks, np.uint8)).cuda()
            img = torch.empty(max(16, plan.bscale_image_bytes(operand)), dtype=torch.uint8, device="cuda")
            plan.preshuffle_bscale(operand, src.data_ptr(), img.data_ptr(), s)
            imgs.append((src, img))
        plan.run_mx(A.data_ptr(), imgs[0][1].data_ptr(), Bx.data_ptr(), imgs[1][1].data_ptr(), C.data_ptr(),
                    stream=s, scale_a=keep["scale_a"].data_ptr() if "scale_a" in keep else None,
                    scale_a_per_row=np.ndim(e.get("scale_a")) > 0,
                    scale_b=keep["scale_b"].data_ptr() if "scale_b" in keep else None,
                    scale_b_per_col=np.ndim(e.get("scale_b")) > 0,
                    bias=keep["bias"].data_ptr() if "bias" in keep else None,
                    epilogue=tg.EPILOGUES[e.get("kind", "none")])
    elif workspace is not None and workspace is not False:
        e = dict(epi) if epi is not None else (
            dict(scale_a=scale[0], scale_b=scale[1], kind="none") if use_scale else dict(kind="none"))
        keep = {k: _dev_f32(e[k]) for k in ("scale_a", "scale_b", "bias") if e.get(k) is not None}
        wsb = plan.workspace_bytes() if workspace is True else int(workspace)
        W = torch.full((max(16, wsb),), 0x7F, dtype=torch.uint8, device="cuda")   # garbage: never read unwritten
        plan.run_ws(A.data_ptr(), Bx.data_ptr(), C.data_ptr(), W.data_ptr() if wsb else None, wsb, stream=s,
                    scale_a=keep["scale_a"].data_ptr() if "scale_a" in keep else None,
                    scale_a_per_row=np.ndim(e.get("scale_a")) > 0,
                    scale_b=keep["scale_b"].data_ptr() if "scale_b" in keep else None,
                    scale_b_per_col=np.ndim(e.get("scale_b")) > 0,
                    bias=keep["bias"].data_ptr() if "bias" in keep else None,
                    epilogue=tg.EPILOGUES[e.get("kind", "none")])
    elif epi is None:
        sc = torch.tensor(scale, dtype=torch.float32, device="cuda")
        plan.run(A.data_ptr(), Bx.data_ptr(), C.data_ptr(), sc.data_ptr() if use_scale else None, s)
    else:
        keep = {k: _dev_f32(epi[k]) for k in ("scale_a", "scale_b", "bias") if epi.get(k) is not None}
        plan.run_ex(A.data_ptr(), Bx.data_ptr(), C.data_ptr(), stream=s,
                    scale_a=keep["scale_a"].data_ptr() if "scale_a" in keep else None,
                    scale_a_per_row=np.ndim(epi.get("scale_a")) > 0,
                    scale_b=keep["scale_b"].data_ptr() if "scale_b" in keep else None,
                    scale_b_per_col=np.ndim(epi.get("scale_b")) > 0,
                    bias=keep["bias"].data_ptr() if "bias" in keep else None,
                    epilogue=tg.EPILOGUES[epi.get("kind", "none")])
    torch.cuda.synchronize()
    raw = C.cpu().numpy()[:M * N * ob]
    info = plan.info()
    if own:
        plan.close()
    bits = raw.view(np.uint32 if out == "f32" else np.uint16).reshape(M, N)
    return (bits, info) if return_plan_info else bits


def decode(bits: np.ndarray) -> np.ndarray:
    """C bits -> float64 (fp32 or bf16 storage)."""
    if bits.dtype == np.uint32:
        return bits.view(np.float32).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_within_bound(C: np.ndarray, C_ref: np.ndarray, S: np.ndarray, dtype: str, what: str = ""):
    assert np.all(np.isfinite(C)), "%s: non-finite output" % what
    err = np.abs(C - C_ref)
    bound = ABS_COEF * S + RHO[dtype] * np.abs(C_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join("(%s) got %r want %r bound %r" % (tuple(i), C[tuple(i)], C_ref[tuple(i)],
                                                             bound[tuple(i)]) for i in idx)
        raise AssertionError("%s: %d of %d elements outside the bound; %s" % (what, int(bad.sum()), bad.size, detail))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def assert_epilogue_within_bound(Y, Y_ref, S_z, Z_abs, bias_abs, dtype, kind, what=""):
    """Bound for C = act((acc * sa) * sb + bias):
    |Y - Y_ref| <= L * (4e-6 * S_z + 2^-20 * (Z_abs + bias_abs)) + rho * |Y_ref|,
    with S_z = |sa * sb| * sum_k |a_ik b_jk| (the GEMM's own term, scaled),
    Z_abs = |(acc * sa) * sb| of the exact result, L the activation's largest
    slope (carries the pre-activation error through), 2^-20 covering the fp32
    roundings of the scale, bias and activation evaluation, and rho the output
    rounding term of the GEMM bound."""
    import oracle
    assert np.all(np.isfinite(Y)), "%s: non-finite output" % what
    L = oracle.ACT_LIPSCHITZ[kind]
    bound = L * (ABS_COEF * S_z + 2.0 ** -20 * (Z_abs + bias_abs)) + RHO[dtype] * np.abs(Y_ref)
    err = np.abs(Y - Y_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join("(%s) got %r want %r bound %r" % (tuple(i), Y[tuple(i)], Y_ref[tuple(i)],
                                                             bound[tuple(i)]) for i in idx)
        raise AssertionError("%s: %d of %d elements outside the bound; %s" % (what, int(bad.sum()), bad.size, detail))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def block_entries(M: int, N: int, seed: int, block: int = 16):
    """Entries of C to check at full size: one in every block x block tile,
    at a seeded random position inside the tile (so each of the 256 positions
    of a 16 x 16 MFMA output fragment is hit about M * N / 65536 times, and
    every tile of every workgroup, wave and MFMA is visited), plus rows 0 and
    M - 1 and columns 0 and N - 1 in full."""
    rng = np.random.default_rng(seed)
    bm, bn = -(-M // block), -(-N // block)
    slot = rng.integers(0, block * block, size=(bm, bn))
    r = np.minimum(np.arange(bm)[:, None] * block + slot // block, M - 1).reshape(-1)
    c = np.minimum(np.arange(bn)[None, :] * block + slot % block, N - 1).reshape(-1)
    rows = [np.zeros(N, np.int64), np.full(N, M - 1, np.int64), np.arange(M), np.arange(M), r]
    cols = [np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1, np.int64), c]
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def force(kernel=None, splits=0):
    """Set the kernel choice (a name of tg.KERNELS, None = the planner's) and
    split count of the plans created by run_gemm and plan(); the plan_opts
    fixture restores the defaults after each test."""
    PLAN_OPTS["kernel"] = tg.KERNELS[kernel or "auto"]
    PLAN_OPTS["splits"] = int(splits)


def plan(M, N, K, dtype_code, layout_code):
    """A tg.Plan with the current PLAN_OPTS (kernel choice, split count)."""
    return tg.Plan(M, N, K, dtype_code, layout_code, **PLAN_OPTS)
