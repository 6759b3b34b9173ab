"""A whole muon_step_batched call captured in a HIP graph (torch.cuda.graph on
the current stream) and replayed: the library only enqueues kernels -- no
allocation, memset or synchronisation -- so a captured step must give, replay
after replay, bit for bit what the same number of eager steps gives.  Every
replay is checked, with eager work and a synchronisation between replays."""

import sys

import pytest
import torch

from matrix_optimizer_02_amd import dmuon_ns as d
from matrix_optimizer_02_amd.workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

# wide and tall bf16 (Gram space), square (short side) and an fp32-path matrix
SHAPES = [(256, 768), (768, 256), (384, 384), (128, 640), (200, 72)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_captured_step_replays_match_eager_steps():
    w = custom_workload("graph", SHAPES, "bf16", "bf16")
    G, M, W = make_inputs(w, "cuda", seed=8)
    G.append(torch.randn(96, 160, device="cuda") * 1e-3)   # fp32 gradient
    M.append(torch.zeros(96, 160, device="cuda"))
    W.append(torch.randn(96, 160, device="cuda") * 0.02)
    Mg, Wg = [x.clone() for x in M], [x.clone() for x in W]
    plan = d.plan_for(G, [x.dtype for x in W])
    ws_e, ws_g = d.workspace_for(plan), d.workspace_for(plan)

    say("case graph capture of muon_step_batched, 3 replays")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            d.muon_step_batched(plan, G, Mg, Wg, workspace=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(3):
        d.muon_step_batched(plan, G, M, W, workspace=ws_e)  # eager step k
        graph.replay()
        junk = torch.randn(1 << 20, device="cuda").sum()      # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i in range(len(G)):
            assert torch.equal(M[i], Mg[i]), (k, i)
            assert torch.equal(W[i].view(torch.int16) if W[i].dtype == torch.bfloat16 else W[i],
                               Wg[i].view(torch.int16) if Wg[i].dtype == torch.bfloat16 else Wg[i]), (k, i)
        say(f"  replay {k}: bit-identical to eager step {k}")
