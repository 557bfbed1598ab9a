"""gemm_run_ws_noalloc (the split-K entry point on the library's static
workspace) against gemm_run_ws with a caller-provided workspace.

Both run the same tile kernel with the same K slices and the same ordered
reduction, so C must agree bit for bit.  Two calls in a row, the second on a
smaller problem, show that what the first call leaves in the shared array
does not leak into the second.  The second problem has integer-valued
inputs, so it is also compared bit for bit with the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import tiled_gemm_amd as tg
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _dev(bits):
    bits = np.ascontiguousarray(bits)
    return torch.from_numpy(bits.view(np.int16) if bits.dtype == np.uint16 else bits).cuda()


def _run_both(M, N, K, layout, inp, scale_a, scale_b):
    """C from gemm_run_ws_noalloc and from gemm_run_ws, as raw bf16 bits."""
    s = torch.cuda.current_stream().cuda_stream
    with tg.Plan(M, N, K, tg.GEMM_BF16_OUT_BF16, tg.LAYOUTS[layout]) as p:
        info = p.info()
        need = p.workspace_bytes()
        assert info["ws_splits"] > 1 and 0 < need <= tg.GEMM_STATIC_WORKSPACE_BYTES
        A, B = _dev(inp.A), _dev(inp.B)
        if layout == "bt_preshuffled":
            Bs = torch.empty(tg.gemm_preshuffled_b_bytes(p.handle), dtype=torch.uint8, device="cuda")
            p.preshuffle_b(B.data_ptr(), Bs.data_ptr(), s)
            B = Bs
        sa = torch.tensor([scale_a], dtype=torch.float32, device="cuda")
        sb = torch.tensor([scale_b], dtype=torch.float32, device="cuda")
        C0 = torch.full((M * N,), 0x5A5A, dtype=torch.int16, device="cuda")
        C1 = torch.full((M * N,), 0x2B2B, dtype=torch.int16, device="cuda")
        Wk = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        p.run_ws_noalloc(A.data_ptr(), B.data_ptr(), C0.data_ptr(), stream=s, scale_a=sa.data_ptr(),
                         scale_b=sb.data_ptr())
        p.run_ws(A.data_ptr(), B.data_ptr(), C1.data_ptr(), Wk.data_ptr(), need, stream=s,
                 scale_a=sa.data_ptr(), scale_b=sb.data_ptr())
        torch.cuda.synchronize()
        return (C0.cpu().numpy().view(np.uint16).reshape(M, N), C1.cpu().numpy().view(np.uint16).reshape(M, N),
                info)


def test_noalloc_matches_workspace_entry_point(oracle_mod):
    # first call: random bf16, 32 MiB of partials (4 slices)
    M, N, K = 512, 4096, 4096
    say("case noalloc first", M, N, K)
    w = W.WORKLOADS["bf16_4096"]
    inp = W.make_inputs(w, M=M, N=N, K=K, seed=91)
    got, want, info = _run_both(M, N, K, "bt_preshuffled", inp, 1.0, 1.0)
    say("  splits", info["ws_splits"])
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first call: %d mismatches, first %s" % (len(bad), bad[:3].tolist())
    # second call, smaller: integer-valued inputs, exact in fp32
    M, N, K = 200, 1024, 2048
    say("case noalloc second", M, N, K)
    inp = W.int_inputs(M, N, K, "bf16", seed=92)
    got, want, info = _run_both(M, N, K, "bt", inp, 0.5, 2.0)
    say("  splits", info["ws_splits"])
    bad = np.argwhere(got != want)
    assert bad.size == 0, "second call: %d mismatches, first %s" % (len(bad), bad[:3].tolist())
    C_ref, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype="bf16", sigma=1.0, want_s=False)
    assert np.array_equal(got, oracle_mod.round_bf16(C_ref))


def test_noalloc_refuses_partials_above_the_static_workspace():
    # 4 forced slices of 1024 x 8192 fp32 partials: 128 MiB > 64 MiB
    with tg.Plan(1024, 8192, 8192, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, splits=4) as p:
        assert p.workspace_bytes() > tg.GEMM_STATIC_WORKSPACE_BYTES
        A = torch.empty(16, dtype=torch.uint8, device="cuda")
        with pytest.raises(tg.GemmError, match="static workspace"):
            p.run_ws_noalloc(A.data_ptr(), A.data_ptr() + 4096, A.data_ptr() + 8192)


def test_noalloc_without_split_is_gemm_run_ex(oracle_mod):
    M, N, K = 256, 512, 1024                   # plans without a split need no workspace
    inp = W.int_inputs(M, N, K, "bf16", seed=93)
    s = torch.cuda.current_stream().cuda_stream
    with tg.Plan(M, N, K, tg.GEMM_BF16_OUT_BF16, tg.GEMM_LAYOUT_BT, splits=1) as p:
        assert p.workspace_bytes() == 0
        A, B = _dev(inp.A), _dev(inp.B)
        C = torch.full((M * N,), 0x5A5A, dtype=torch.int16, device="cuda")
        p.run_ws_noalloc(A.data_ptr(), B.data_ptr(), C.data_ptr(), stream=s)
        torch.cuda.synchronize()
    C_ref, _ = oracle_mod.gemm_bt(inp.A, inp.B, dtype="bf16", want_s=False)
    assert np.array_equal(C.cpu().numpy().view(np.uint16).reshape(M, N), oracle_mod.round_bf16(C_ref))
