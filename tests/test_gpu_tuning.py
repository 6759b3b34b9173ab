"""GPU checks of the per-shape configurations (tuning entries) and of
muon_autotune, through the C ABI, against the fp64 oracle.

* The XCD remap only changes which workgroup computes which tile, so every
  remap choice gives bit-identical outputs.
* Tile 128 on buckets whose default tile is 256, and either form of the
  recurrence, meet the bf16 bar (relative Frobenius error <= 2e-2).
* muon_autotune returns one valid entry per bucket with a measured cost, and a
  plan built from them meets the same bar.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from matrix_optimizer_02_amd import dmuon_ns as d
from matrix_optimizer_02_amd.workloads import custom_workload, host_tensor, GRAD

pytestmark = pytest.mark.gpu

A, B, C = oracle.NS_COEFFS
EPS = 1e-7
TOL = 2e-2
SHAPES = [(256, 1536), (1536, 256), (512, 768), (768, 512), (1024, 1536), (384, 1000), (128, 640), (256, 256)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def inputs(seed=4):
    w = custom_workload("tuning", SHAPES, "bf16", "bf16", g_std=1.0)
    return [host_tensor(w, i, GRAD, seed=seed).cuda() for i in range(w.count)]


def orth(plan, xs):
    ws = d.workspace_for(plan)
    outs = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in xs]
    d.ns_orthogonalize_batched(plan, xs, outs, workspace=ws)
    torch.cuda.synchronize()
    return outs


def entries_for(xs, **over):
    """The default plan's bucket configs with fields overridden where allowed."""
    base = d.plan_for(xs, [torch.float32] * len(xs))
    out = []
    for b in range(base.info()[1]):
        e = base.config(b)
        for k, v in over.items():
            if k == "tile" and (e.padded_m % v or e.padded_n % v):
                continue
            # square buckets keep the short side (the Gram space resolves their
            # small singular values worse; the automatic rule never picks it there)
            if k == "algo" and v == d.ALGO_GRAM_SPACE and e.padded_m == e.padded_n:
                continue
            setattr(e, k, v)
        out.append(e)
    return out


def test_remap_choices_are_bit_identical():
    xs = inputs()
    say("case tuning: XCD remap 0 / 4 / 15, default tiles")
    runs = [orth(d.plan_for(xs, [torch.float32] * len(xs), tuning=entries_for(xs, xcd_remap=m)), xs)
            for m in (0, 4, 15)]
    for i in range(len(xs)):
        for r in runs[1:]:
            assert torch.equal(runs[0][i].view(torch.int32), r[i].view(torch.int32)), SHAPES[i]


@pytest.mark.parametrize("algo", [d.ALGO_SHORT_SIDE, d.ALGO_GRAM_SPACE])
def test_tile_128_and_forms_meet_the_bar(algo):
    xs = inputs()
    say(f"case tuning: tile 128 everywhere, algo {algo}, remap 15")
    plan = d.plan_for(xs, [torch.float32] * len(xs), tuning=entries_for(xs, tile=128, algo=algo, xcd_remap=15))
    for b in range(plan.info()[1]):
        assert plan.bucket(b).tile == 128
    outs = orth(plan, xs)
    for i, x in enumerate(xs):
        e = rel(f64(outs[i]), oracle.newton_schulz(f64(x), 5, A, B, C, EPS))
        assert e < TOL, (SHAPES[i], e)


def test_autotune_entries_and_parity(tmp_path):
    xs = inputs(seed=5)
    say("case muon_autotune on the tuning shape set, reps 1")
    ents = d.autotune(xs, reps=1)
    plan0 = d.plan_for(xs, [torch.float32] * len(xs))
    assert len(ents) == plan0.info()[1]
    for b, e in enumerate(ents):
        c = plan0.config(b)
        assert (e.path, e.padded_m, e.padded_n) == (c.path, c.padded_m, c.padded_n)
        assert e.tile in (128, 256) and e.padded_m % e.tile == 0 and e.padded_n % e.tile == 0
        assert e.algo in (d.ALGO_SHORT_SIDE, d.ALGO_GRAM_SPACE) and e.xcd_remap in (0, 4, 15)
        # the Gram space is only tried where the automatic rule allows it
        assert e.algo == d.ALGO_SHORT_SIDE or c.algo == d.ALGO_GRAM_SPACE
        assert e.cost_ms_per_matrix > 0
        say(f"  {e}")
    path = str(tmp_path / "tune.json")
    d.save_tuning(ents, path)
    loaded = d.load_tuning(path)
    plan = d.plan_for(xs, [torch.float32] * len(xs), tuning=loaded)
    outs = orth(plan, xs)
    for i, x in enumerate(xs):
        e = rel(f64(outs[i]), oracle.newton_schulz(f64(x), 5, A, B, C, EPS))
        assert e < TOL, (SHAPES[i], e)


def test_autotune_mixed_small_batch():
    """A batch of small square and wide matrices (the 96-matrix small-batch
    shapes at a third of the count): the entries are valid whichever form the
    whole-batch check keeps, square buckets stay on the short side, and a plan
    from them meets the bar."""
    shapes = [(128, 128)] * 11 + [(128, 512)] * 11 + [(512, 128)] * 11
    w = custom_workload("tuning_small", shapes, "bf16", "bf16", g_std=1.0)
    xs = [host_tensor(w, i, GRAD, seed=6).cuda() for i in range(w.count)]
    say("case muon_autotune on a mixed small batch, reps 2")
    ents = d.autotune(xs, reps=2)
    assert len(ents) == d.plan_for(xs, [torch.float32] * len(xs)).info()[1]
    for e in ents:
        say(f"  {e}")
        assert e.cost_ms_per_matrix > 0 and e.tile == 128
        if e.padded_m == e.padded_n:
            assert e.algo == d.ALGO_SHORT_SIDE
    plan = d.plan_for(xs, [torch.float32] * len(xs), tuning=ents)
    outs = orth(plan, xs)
    for i, x in enumerate(xs):
        e = rel(f64(outs[i]), oracle.newton_schulz(f64(x), 5, A, B, C, EPS))
        assert e < TOL, (shapes[i], e)
