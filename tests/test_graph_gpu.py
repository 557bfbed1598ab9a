"""The GEMM paths under HIP graph capture.

The entry points allocate nothing and record no memsets, so a caller can
capture them.  Each case runs once eagerly, is captured into a graph (torch's
capture stream is the launch stream), and is replayed three times with eager
work and synchronisations between the replays; every replay must reproduce the
eager result bit for bit (the kernels are deterministic).
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


# (name, M, N, K, layout, use the workspace entry point, expected kernel)
CASES = [
    ("pipelined 256x256", 4096, 4096, 512, "bt_preshuffled", False, 0),
    ("split K", 256, 2048, 4096, "bt", True, 0),
    ("skinny", 32, 2048, 4096, "bt_preshuffled", False, 1),
]


@pytest.mark.parametrize("name,M,N,K,layout,ws,kernel", CASES)
def test_graph_replays_match_eager(name, M, N, K, layout, ws, kernel):
    say("case graph", name, M, N, K, layout)
    inp = W.make_inputs(W.WORKLOADS["bf16_4096"], M=M, N=N, K=K, seed=M + N + K)
    A = torch.from_numpy(inp.A.view(np.int16)).cuda()
    B = torch.from_numpy(inp.B.view(np.int16)).cuda()
    plan = tg.Plan(M, N, K, tg.GEMM_BF16_OUT_BF16, tg.LAYOUTS[layout])
    info = plan.info()
    assert info["kernel"] == kernel
    if ws:
        assert info["ws_splits"] > 1
    s0 = torch.cuda.current_stream().cuda_stream
    Bx = B
    if layout == "bt_preshuffled":
        Bx = torch.empty(tg.gemm_preshuffled_b_bytes(plan.handle), dtype=torch.uint8, device="cuda")
        plan.preshuffle_b(B.data_ptr(), Bx.data_ptr(), s0)
    wsb = plan.workspace_bytes() if ws else 0
    Wk = torch.empty(max(16, wsb), dtype=torch.uint8, device="cuda")
    C_eager = torch.empty(M * N, dtype=torch.int16, device="cuda")
    C_graph = torch.empty(M * N, dtype=torch.int16, device="cuda")

    def launch(C, stream):
        if ws:
            plan.run_ws(A.data_ptr(), Bx.data_ptr(), C.data_ptr(), Wk.data_ptr(), wsb, stream=stream)
        else:
            plan.run(A.data_ptr(), Bx.data_ptr(), C.data_ptr(), None, stream)

    launch(C_eager, s0)
    torch.cuda.synchronize()
    want = C_eager.cpu().numpy()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(C_graph, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(3):
        C_graph.fill_(0x5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C_graph.cpu().numpy()
        assert np.array_equal(got, want), "replay %d differs from the eager result in %d outputs" % (
            r, int((got != want).sum()))
        launch(C_eager, s0)                     # eager work between the replays
        torch.cuda.synchronize()
    del g
    plan.close()
