"""GPU checks of the update written by the kernel that ends the iteration.

By default the resident kernel writes the update (or, for the orthogonalisation
entry point, the output) of every member of a resident bucket, and the last
B X launch's epilogue that of every bf16 parameter whose bucket runs the tiled
bf16 products and whose cols is a multiple of 8; the apply pass writes the
others.  A tuning entry with apply_pass = 1 sends every member of its bucket
through the apply pass instead.  Both routes compute W' = W (1 - lr wd) -
lr s O from the same bf16 O, so they must agree bit for bit; the oracle parity
of the default route is covered by the step tests.  The resident kernel also
sums the norm partials itself, so its matrices' normalisation is checked
against the separate finalize pass here as well.

The tiled set mixes wide and tall (transposed) matrices, ragged sides,
Gram-space and short-side buckets and tile 128 and 256, with an fp32 parameter
and a tall matrix whose cols is not a multiple of 8 (those two take the apply
pass either way).  The resident buckets (padded 128 x 128, 128 x 256 and
128 x 384 or 128 x 512) hold wide and tall matrices with bf16 and fp32
parameters, with cols a multiple of 8 (16-byte chunks) and not (element by
element).
"""

import sys

import pytest
import torch

from matrix_optimizer_02_amd import dmuon_ns as d
from matrix_optimizer_02_amd.workloads import GRAD, MOMENTUM, PARAM, custom_workload, host_tensor

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 4096, "bf16"), (4096, 1024, "bf16"), (300, 520, "bf16"), (520, 300, "bf16"),
          (1000, 384, "bf16"), (384, 1000, "f32"), (2048, 2048, "bf16"), (128, 640, "bf16"),
          (640, 128, "bf16"), (264, 136, "bf16"),
          # resident buckets
          (100, 250, "bf16"), (250, 100, "bf16"), (120, 256, "bf16"), (250, 100, "f32"), (128, 512, "f32"),
          (384, 96, "f32"), (512, 128, "bf16"), (128, 128, "bf16"), (77, 77, "f32")]
RESIDENT = SHAPES[10:]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(seed=11):
    wb = custom_workload("fused", [(r, c) for r, c, _ in SHAPES], "bf16", "bf16", g_std=1e-3, w_std=0.02)
    wf = custom_workload("fused", [(r, c) for r, c, _ in SHAPES], "bf16", "f32", g_std=1e-3, w_std=0.02)
    G, M, W = [], [], []
    for i, (_, _, pd) in enumerate(SHAPES):
        w = wb if pd == "bf16" else wf
        G.append(host_tensor(w, i, GRAD, seed).cuda())
        M.append(host_tensor(w, i, MOMENTUM, seed).cuda())
        W.append(host_tensor(w, i, PARAM, seed).cuda())
    return G, M, W


def plans(G, W, check_routes=False):
    fused = d.plan_for(G, [w.dtype for w in W])
    if check_routes:
        for i, (r, c, pd) in enumerate(SHAPES):
            resident = fused.bucket(fused.query(i).bucket).resident
            assert resident == ((r, c, pd) in RESIDENT), (r, c, pd)
            assert fused.update_fused(i) == (resident or (pd == "bf16" and c % 8 == 0)), (r, c, pd)
    entries = []
    for b in range(fused.info()[1]):
        e = fused.config(b)
        e.apply_pass = 1
        entries.append(e)
    separate = d.plan_for(G, [w.dtype for w in W], tuning=entries)
    for b in range(separate.info()[1]):
        assert separate.config(b).apply_pass == 1 and fused.config(b).apply_pass == 0
    return fused, separate


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("steps", [5, 1, 2])
def test_fused_update_matches_the_apply_pass_bitwise(steps):
    G, M0, W0 = inputs()
    fused, separate = plans(G, W0, check_routes=True)
    out = {}
    for name, plan in (("fused", fused), ("separate", separate)):
        say(f"case fused update: step, {name} plan, ns_steps {steps}")
        M = [m.clone() for m in M0]
        W = [w.clone() for w in W0]
        d.muon_step_batched(plan, G, M, W, weight_decay=0.01, ns_steps=steps, workspace=d.workspace_for(plan))
        torch.cuda.synchronize()
        out[name] = (M, W)
    for i, (r, c, pd) in enumerate(SHAPES):
        assert torch.equal(bits(out["fused"][1][i]), bits(out["separate"][1][i])), (r, c, pd)
        assert torch.equal(out["fused"][0][i].view(torch.int32), out["separate"][0][i].view(torch.int32)), (r, c)
        # the update moved every parameter
        assert not torch.equal(bits(out["fused"][1][i]), bits(W0[i])), (r, c, pd)


def test_fused_output_matches_the_apply_pass_bitwise():
    G, _, W0 = inputs(seed=12)
    fused, separate = plans(G, W0)
    res = {}
    for name, plan in (("fused", fused), ("separate", separate)):
        say(f"case fused update: orthogonalisation, {name} plan")
        outs = [torch.full_like(w, float("nan")) for w in W0]
        d.ns_orthogonalize_batched(plan, G, outs, workspace=d.workspace_for(plan))
        torch.cuda.synchronize()
        res[name] = outs
    for i, (r, c, pd) in enumerate(SHAPES):
        assert torch.equal(bits(res["fused"][i]), bits(res["separate"][i])), (r, c, pd)
        assert torch.isfinite(res["fused"][i].float()).all(), (r, c, pd)


def test_fused_plan_runs_no_apply_pass():
    # four 4096 x 4096 bf16 matrices: the apply pass moves 6 bytes per element
    # (about 0.4 GB); with the update fused, nothing runs after the last B X
    shapes = [(4096, 4096)] * 4
    w = custom_workload("fused_timing", shapes, "bf16", "bf16")
    G = [host_tensor(w, i, GRAD, 0).cuda() for i in range(len(shapes))]
    M = [host_tensor(w, i, MOMENTUM, 0).cuda() for i in range(len(shapes))]
    W = [host_tensor(w, i, PARAM, 0).cuda() for i in range(len(shapes))]
    fused, separate = plans(G, W)
    apply_ms = {}
    for name, plan in (("fused", fused), ("separate", separate)):
        say(f"case fused update: apply-phase time, {name} plan")
        ws = d.workspace_for(plan)
        ev = d.PhaseEvents(5)
        times = []
        for _ in range(3):
            d.muon_step_batched_profiled(plan, G, M, W, ev, workspace=ws)
            torch.cuda.synchronize()
            times.append(ev.elapsed_ms()[-1])
        ev.close()
        apply_ms[name] = min(times)
    say(f"  apply phase ms: {apply_ms}")
    assert apply_ms["separate"] > 0.02
    assert apply_ms["fused"] < 0.25 * apply_ms["separate"]
