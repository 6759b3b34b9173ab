"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances (relative Frobenius error unless stated):
  * Newton-Schulz output O: 1e-4 on the fp32 path, 2e-2 on the bf16-MFMA path;
  * momentum M': 1e-6 (one fp32 rounding plus fp32(beta) vs beta);
  * updated parameters W': derived from the arithmetic, per matrix
        ||W'_gpu - W'_ref|| <= 0.5 (1 + 2^-8) ||ulp(W'_ref)|| + lr s tol_O ||O_ref||
    i.e. the unavoidable rounding of the stored parameter plus the O tolerance
    carried through the update (triangle inequality, element by element).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from matrix_optimizer_02_amd import dmuon_ns as d
from matrix_optimizer_02_amd.workloads import (custom_workload, get_workload, host_tensor,
                                                make_inputs, GRAD, MOMENTUM, PARAM)

pytestmark = pytest.mark.gpu

A, B, C = oracle.NS_COEFFS
LR, BETA, EPS = 0.02, 0.95, 1e-7
TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def ulp(x, dtype):
    """Spacing of the dtype at |x| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - bits, -126 - bits + 1))


def check_param(Wn_gpu, W0, out_ref, dtype, path, rows, cols):
    Wn_ref = out_ref["W_new"]
    q = 0.5 * (1 + 2.0 ** -8) * np.linalg.norm(ulp(Wn_ref, dtype))
    s = oracle.update_scale(rows, cols)
    bound = q + LR * s * TOL[path] * np.linalg.norm(out_ref["O"])
    err = np.linalg.norm(Wn_gpu - Wn_ref)
    assert err <= bound, (err, bound)


def step_gpu(w, seed=0, param_dtype=None, zero_params=False, ns_steps=5, steps=1, algo="auto", restart=0):
    """Run ``steps`` fused steps on a workload; returns host inputs and outputs."""
    G, M, W = make_inputs(w, "cuda", seed)
    if param_dtype is not None or zero_params:
        pd = param_dtype or torch.float32
        W = [torch.zeros_like(x, dtype=pd) if zero_params else x.to(pd) for x in W]
    host = {"G": [f64(x) for x in G], "M": [f64(x) for x in M], "W": [f64(x) for x in W]}
    plan = d.plan_for(G, [x.dtype for x in W], algo, restart)
    ws = d.workspace_for(plan)
    for _ in range(steps):
        d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, ns_steps=ns_steps, workspace=ws)
    torch.cuda.synchronize()
    return host, {"M": [f64(x) for x in M], "W": [f64(x) for x in W]}, G, M, W


def orth_gpu(inputs, out_dtype=torch.float32, ns_steps=5, eps=EPS, algo="auto", restart=0):
    plan = d.plan_for(inputs, [out_dtype] * len(inputs), algo, restart)
    ws = d.workspace_for(plan)
    outs = [torch.empty(x.shape, dtype=out_dtype, device="cuda") for x in inputs]
    d.ns_orthogonalize_batched(plan, inputs, outs, ns_steps=ns_steps, eps=eps, workspace=ws)
    torch.cuda.synchronize()
    return outs


# ---- the single fp32 matrix (256 x 512, N(0,1), zero momentum) ----------------------

def test_f32_single_matrix_step():
    w = get_workload("f32_256x512")
    say("case f32_256x512 muon_step_batched seed 0")
    host, out, *_ = step_gpu(w)
    ref = oracle.muon_step(host["G"][0], host["M"][0], host["W"][0], lr=LR, beta=BETA, eps=EPS)
    assert rel(out["M"][0], ref["M_new"]) < 1e-6
    upd_gpu = out["W"][0] - host["W"][0]
    upd_ref = ref["W_new"] - host["W"][0]
    assert rel(upd_gpu, upd_ref) < TOL["f32"]
    check_param(out["W"][0], host["W"][0], ref, "f32", "f32", 256, 512)


def test_f32_single_matrix_orthogonalize():
    w = get_workload("f32_256x512")
    G = host_tensor(w, 0, GRAD).cuda()
    say("case f32_256x512 ns_orthogonalize_batched")
    for steps in (0, 1, 5):
        O = f64(orth_gpu([G], ns_steps=steps)[0])
        ref = oracle.newton_schulz(f64(G), steps, A, B, C, EPS)
        assert rel(O, ref) < TOL["f32"], steps


# ---- the 96-matrix bf16 batch ---------------------------------------------------------

def test_small_batch_step_bf16_params():
    w = get_workload("bf16_small_batch_96")
    say("case bf16_small_batch_96 muon_step_batched bf16 params")
    host, out, *_ = step_gpu(w)
    for i, spec in enumerate(w.matrices):
        ref = oracle.muon_step(host["G"][i], host["M"][i], host["W"][i], lr=LR, beta=BETA, eps=EPS)
        assert rel(out["M"][i], ref["M_new"]) < 1e-6, i
        check_param(out["W"][i], host["W"][i], ref, "bf16", "bf16", spec.rows, spec.cols)


@pytest.mark.parametrize("algo", ["auto", "short_side"])
def test_small_batch_step_recovers_O(algo):
    # W = 0 in fp32: W' = -lr s O exposes the step's own orthogonalised update
    w = get_workload("bf16_small_batch_96")
    say(f"case bf16_small_batch_96 muon_step_batched fp32 zero params, {algo}")
    host, out, *_ = step_gpu(w, zero_params=True, algo=algo)
    errs = []
    for i, spec in enumerate(w.matrices):
        ref = oracle.muon_step(host["G"][i], host["M"][i], host["W"][i], lr=LR, beta=BETA, eps=EPS)
        s = oracle.update_scale(spec.rows, spec.cols)
        errs.append(rel(-out["W"][i] / (LR * s), ref["O"]))
    say("max rel O error", max(errs))
    assert max(errs) < TOL["bf16"]


# ---- ragged shapes, several tiles, both paths ------------------------------------------

SHAPE_SETS = {
    "bf16_ragged": ([(300, 700), (700, 300), (129, 257), (1000, 130), (64, 64), (1, 513), (513, 1),
                     (128, 128), (200, 72)], "bf16"),
    "bf16_multi_tile": ([(1024, 1536), (1536, 1024), (768, 768), (520, 1300)], "bf16"),
    "f32_ragged": ([(70, 33), (33, 70), (200, 200), (1, 65), (130, 250), (1, 1)], "f32"),
}


# the default (Gram space on the buckets with padded n > padded m) and the short side forced
@pytest.mark.parametrize("algo", ["auto", "short_side"])
@pytest.mark.parametrize("name", sorted(SHAPE_SETS))
@pytest.mark.parametrize("ns_steps", [0, 1, 2, 5])
def test_orthogonalize_shapes(name, ns_steps, algo):
    shapes, dt = SHAPE_SETS[name]
    w = custom_workload(name, shapes, dt, dt, g_std=1.0)
    Gs = [host_tensor(w, i, GRAD, seed=3) for i in range(w.count)]
    say(f"case {name} ns_orthogonalize_batched ns_steps={ns_steps} {algo}")
    outs = orth_gpu([g.cuda() for g in Gs], ns_steps=ns_steps, algo=algo)
    for i, g in enumerate(Gs):
        ref = oracle.newton_schulz(f64(g), ns_steps, A, B, C, EPS)
        assert rel(f64(outs[i]), ref) < TOL[dt], (shapes[i], rel(f64(outs[i]), ref))


# every padded long side the resident kernel takes (128 .. 512), wide, tall, square,
# ragged, single-row and 1 x 1
RESIDENT_SHAPES = [(128, 128), (100, 250), (77, 300), (120, 512), (512, 128), (300, 77), (1, 200), (64, 64),
                   (128, 384), (37, 129), (1, 1)]


@pytest.mark.parametrize("ns_steps", [1, 2, 5])
def test_resident_buckets(ns_steps):
    w = custom_workload("resident", RESIDENT_SHAPES, "bf16", "bf16", g_std=1.0)
    Gs = [host_tensor(w, i, GRAD, seed=12) for i in range(w.count)]
    dev = [g.cuda() for g in Gs]
    plan = d.plan_for(dev, [torch.float32] * len(dev))
    assert all(plan.bucket(b).resident for b in range(plan.info()[1]))
    say(f"case resident buckets ns_orthogonalize_batched ns_steps={ns_steps}")
    outs = orth_gpu(dev, ns_steps=ns_steps)
    for i, g in enumerate(Gs):
        ref = oracle.newton_schulz(f64(g), ns_steps, A, B, C, EPS)
        assert rel(f64(outs[i]), ref) < TOL["bf16"], (RESIDENT_SHAPES[i], rel(f64(outs[i]), ref))


# More buckets than one grouped launch's segment table holds (24): 30 bf16 shapes
# that pad to 30 distinct (m, n) buckets, wide and tall alternating, so every
# phase of the 256-tile class goes out as two launches, in either form of the
# recurrence (the default keeps these short sides below 1024 on the short side;
# the Gram space is forced on all of them once), and 26 fp32 shapes do the same
# for the fp32 class.
MANY_BF16 = [((m, n) if k % 2 == 0 else (n, m))
             for k, (m, n) in enumerate((m, n_pad - 37) for m, base in ((140, 256), (300, 512), (520, 768))
                                        for n_pad in range(base, base + 2560, 256))]
MANY_F32 = [(m, m + 64 * j + 5) for m in (40, 100) for j in range(13)]


@pytest.mark.parametrize("path,algo", [("bf16", "auto"), ("bf16", "gram_space"), ("f32", "auto")])
def test_more_buckets_than_one_launch_holds(path, algo):
    shapes = MANY_BF16 if path == "bf16" else MANY_F32
    w = custom_workload(f"many_{path}", shapes, path, "f32")
    say(f"case {len(shapes)} buckets ({path}, {algo}) muon_step_batched fp32 zero params")
    host, out, G, *_ = step_gpu(w, seed=21, zero_params=True, algo=algo)
    plan = d.plan_for(G, [torch.float32] * len(G), algo)
    assert plan.info()[1] == len(shapes) > 24
    if path == "bf16":
        algos = {plan.bucket(b).algo for b in range(plan.info()[1])}
        assert algos == {d.ALGO_GRAM_SPACE if algo == "gram_space" else d.ALGO_SHORT_SIDE}
    for i, (r, c) in enumerate(shapes):
        ref = oracle.muon_step(host["G"][i], host["M"][i], host["W"][i], lr=LR, beta=BETA, eps=EPS)
        s_upd = oracle.update_scale(r, c)
        assert rel(out["M"][i], ref["M_new"]) < 1e-6, (r, c)
        e = rel(-out["W"][i] / (LR * s_upd), ref["O"])
        assert e < TOL[path], ((r, c), e)


@pytest.mark.parametrize("name", sorted(SHAPE_SETS))
def test_step_shapes(name):
    shapes, dt = SHAPE_SETS[name]
    w = custom_workload(name, shapes, dt, dt)
    say(f"case {name} muon_step_batched")
    host, out, *_ = step_gpu(w, seed=5)
    for i, (r, c) in enumerate(shapes):
        ref = oracle.muon_step(host["G"][i], host["M"][i], host["W"][i], lr=LR, beta=BETA, eps=EPS)
        assert rel(out["M"][i], ref["M_new"]) < 1e-6, (r, c)
        check_param(out["W"][i], host["W"][i], ref, dt, dt, r, c)
    # the same gradients and momenta with zero fp32 parameters: W' = -lr s O holds
    # the step's own O to the path's tolerance (the bf16 W' bound above is dominated
    # by the parameter's rounding and would admit a much larger O error)
    say(f"case {name} muon_step_batched fp32 zero params")
    host, out, *_ = step_gpu(w, seed=5, zero_params=True)
    for i, (r, c) in enumerate(shapes):
        ref = oracle.muon_step(host["G"][i], host["M"][i], host["W"][i], lr=LR, beta=BETA, eps=EPS)
        e = rel(-out["W"][i] / (LR * oracle.update_scale(r, c)), ref["O"])
        assert e < TOL[dt], ((r, c), e)


def test_mixed_precision_batch():
    # one call with both paths and both parameter dtypes
    specs = [(300, 500, torch.bfloat16, torch.float32), (256, 384, torch.float32, torch.bfloat16),
             (96, 640, torch.bfloat16, torch.bfloat16), (640, 96, torch.float32, torch.float32)]
    rng = np.random.default_rng(11)
    Gs = [torch.from_numpy(rng.standard_normal((r, c)).astype(np.float32) * 1e-3).to(gd)
          for r, c, gd, _ in specs]
    Ms = [torch.from_numpy(rng.standard_normal((r, c)).astype(np.float32) * 1e-3) for r, c, _, _ in specs]
    Ws = [torch.from_numpy(rng.standard_normal((r, c)).astype(np.float32) * 0.02).to(pd)
          for r, c, _, pd in specs]
    host = [(f64(g), f64(m), f64(w_)) for g, m, w_ in zip(Gs, Ms, Ws)]
    G, M, W = [x.cuda() for x in Gs], [x.cuda() for x in Ms], [x.cuda() for x in Ws]
    plan = d.plan_for(G, [x.dtype for x in W])
    say("case mixed_precision muon_step_batched")
    d.muon_step_batched(plan, G, M, W, workspace=d.workspace_for(plan))
    torch.cuda.synchronize()
    for i, (r, c, gd, pd) in enumerate(specs):
        ref = oracle.muon_step(*host[i], lr=LR, beta=BETA, eps=EPS)
        path = "bf16" if gd == torch.bfloat16 else "f32"
        assert rel(f64(M[i]), ref["M_new"]) < 1e-6
        check_param(f64(W[i]), host[i][2], ref, "bf16" if pd == torch.bfloat16 else "f32", path, r, c)


# ---- degenerate cases, invariances, determinism --------------------------------------


def test_repeated_steps_are_bit_identical():
    """Tiles reach workgroups through per-XCD queues, so which workgroup
    computes which tile changes from run to run, but every output element is
    accumulated by one wave in one k order: three steps on the same inputs agree
    bit for bit.  The set groups a Gram-space bucket (wide and tall matrices)
    and two short-side ones: 666 tiles in a Gram or square launch and over
    2000 in a B X launch, several for every CU."""
    shapes = [(2048, 6144)] * 8 + [(2048, 2048)] * 8 + [(512, 1536)] * 6 + [(6144, 2048)] * 2
    w = custom_workload("repeat", shapes, "bf16", "bf16")
    G, M, W = make_inputs(w, "cuda", seed=11)
    plan = d.plan_for(G, [x.dtype for x in W])
    assert d.ALGO_GRAM_SPACE in [plan.bucket(b).algo for b in range(plan.info()[1])]
    ws = d.workspace_for(plan)
    runs = []
    for rep in range(3):
        say(f"case repeated step {rep}")
        Mr, Wr = [x.clone() for x in M], [x.clone() for x in W]
        d.muon_step_batched(plan, G, Mr, Wr, lr=LR, beta=BETA, eps=EPS, workspace=ws)
        torch.cuda.synchronize()
        runs.append((Mr, Wr))
    for rep in (1, 2):
        for i in range(len(shapes)):
            assert torch.equal(runs[rep][0][i], runs[0][0][i]), (rep, shapes[i])
            assert torch.equal(runs[rep][1][i].view(torch.int16), runs[0][1][i].view(torch.int16)), (rep, shapes[i])

def test_zero_gradient_and_momentum():
    shapes = [(256, 512), (512, 128), (77, 77)]
    G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    M = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    W = [torch.randn(s, device="cuda").to(torch.bfloat16) for s in shapes]
    W0 = [x.clone() for x in W]
    plan = d.plan_for(G, [x.dtype for x in W])
    say("case zero gradient muon_step_batched")
    d.muon_step_batched(plan, G, M, W, workspace=d.workspace_for(plan))
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(W[i], W0[i]) and torch.count_nonzero(M[i]) == 0
    outs = orth_gpu(G)
    assert all(torch.count_nonzero(o) == 0 for o in outs)


def test_non_finite_inputs_propagate():
    """Reading: non-finite values are not masked.  A NaN or an Inf in one
    gradient leaves that matrix's momentum non-finite at that entry only and
    its W' NaN everywhere, as in the oracle; every other matrix of the batch,
    and every other momentum entry, is bit for bit what a clean run gives."""
    shapes = [(256, 768), (768, 256), (200, 72), (128, 128)]
    w = custom_workload("nonfinite", shapes, "bf16", "bf16")
    G, M, W = make_inputs(w, "cuda", seed=3)
    Gc, Mc, Wc = [x.clone() for x in G], [x.clone() for x in M], [x.clone() for x in W]
    planted = {0: (5, 7, float("nan")), 1: (100, 3, float("inf")), 3: (0, 0, float("-inf"))}
    for i, (r, c, v) in planted.items():
        G[i][r, c] = v
    host = [(f64(G[i]), f64(M[i]), f64(W[i])) for i in range(len(shapes))]
    plan = d.plan_for(G, [x.dtype for x in W])
    say("case non-finite gradients muon_step_batched")
    d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, workspace=d.workspace_for(plan))
    d.muon_step_batched(plan, Gc, Mc, Wc, lr=LR, beta=BETA, eps=EPS, workspace=d.workspace_for(plan))
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        if i not in planted:
            assert torch.equal(M[i], Mc[i]) and torch.equal(W[i].view(torch.int16), Wc[i].view(torch.int16))
            continue
        r, c, v = planted[i]
        with np.errstate(invalid="ignore"):  # Inf / Inf in the normalisation
            ref = oracle.muon_step(*host[i], lr=LR, beta=BETA, eps=EPS)
        assert np.isnan(ref["W_new"]).all()
        assert torch.isnan(W[i]).all(), shapes[i]
        Mi = f64(M[i])
        assert (np.isnan(Mi[r, c]) and np.isnan(ref["M_new"][r, c])) or Mi[r, c] == ref["M_new"][r, c] == v
        keep = torch.ones_like(M[i], dtype=torch.bool)
        keep[r, c] = False
        assert torch.equal(M[i][keep], Mc[i][keep])


def test_rank_one_and_diagonal_inputs():
    # Diagonal input (exact zeros off the diagonal stay exact): per-entry p^5 on
    # both paths at the usual tolerances.
    # Rank-1 input, fp32 path only: the iteration amplifies any component in the
    # null space by p'(0)^k = a^k per k remaining steps (a^5 ~ 487), so rounding
    # noise of the first products, ~u sqrt(K) relative with u = 2^-24 and
    # K = 700, reaches ~ a^4 u sqrt(K) ~ 2.2e-4 of the output: the bound used is
    # 4 a^4 u sqrt(K) ~ 9e-4.  On the bf16 path (u = 2^-9) the same noise is
    # pushed into the band and an exactly rank-1 input has no attainable parity.
    r = np.random.default_rng(4)
    u, v = r.standard_normal(300), r.standard_normal(700)
    G1 = np.outer(u, v).astype(np.float32)
    dg = np.zeros((384, 640), np.float32)
    vals = np.linspace(0.05, 1.0, 384).astype(np.float32)
    dg[np.arange(384), np.arange(384)] = vals
    rank1_tol = 4 * A ** 4 * 2.0 ** -24 * math.sqrt(700)
    cases = [(torch.float32, G1, rank1_tol), (torch.float32, dg, TOL["f32"]),
             (torch.bfloat16, dg, TOL["bf16"])]
    for dt, x, tol in cases:
        xin = torch.from_numpy(x).to(dt)
        say(f"case rank1/diagonal ns_orthogonalize_batched {dt} {x.shape}")
        o = orth_gpu([xin.cuda()])[0]
        e = rel(f64(o), oracle.newton_schulz(f64(xin), 5, A, B, C, EPS))
        say(f"  rel err {e:.3e} (tol {tol:.1e})")
        assert e < tol


# ---- other coefficients: the square's b A term folded into the accumulators, or read
# back in the epilogue (c = 0 or |b / c| > 64) ------------------------------------------

OTHER_COEFFS = [(1.5, -0.5, 0.0),          # the cubic iteration: read back
                (1.5, -0.5, 1e-3),         # |b / c| = 500: read back
                (3.0, -3.2, 1.2),          # folded
                (3.4445, -4.7750, 2.0315)]  # the quintic: folded
OTHER_SHAPES = [(768, 768), (520, 1300), (1300, 520), (1024, 3072), (1, 513), (128, 640)]


@pytest.mark.parametrize("algo", ["auto", "short_side"])
@pytest.mark.parametrize("coeffs", OTHER_COEFFS)
def test_other_coefficients(coeffs, algo):
    a, b, c = coeffs
    w = custom_workload("coeffs", OTHER_SHAPES, "bf16", "bf16", g_std=1.0)
    Gs = [host_tensor(w, i, GRAD, seed=11) for i in range(w.count)]
    say(f"case coefficients {coeffs} {algo}")
    inputs = [g.cuda() for g in Gs]
    plan = d.plan_for(inputs, [torch.float32] * len(inputs), algo)
    ws = d.workspace_for(plan)
    outs = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in inputs]
    d.ns_orthogonalize_batched(plan, inputs, outs, ns_steps=5, a=a, b=b, c=c, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
    for i, g in enumerate(Gs):
        e = rel(f64(outs[i]), oracle.newton_schulz(f64(g), 5, a, b, c, EPS))
        say(f"  {OTHER_SHAPES[i]}: rel err {e:.3e}")
        assert e < TOL["bf16"], (coeffs, OTHER_SHAPES[i], e)


# ---- the Gram-space recurrence: restart intervals, conditioning, growth bound ---------

GRAM_SHAPES = [(256, 768), (768, 256), (384, 1000), (128, 640), (72, 200), (512, 1536)]


@pytest.mark.parametrize("restart", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("ns_steps", [1, 2, 3, 4, 5])
def test_gram_space_restart_intervals(restart, ns_steps):
    # every segmentation of up to 5 iterations (the last segment shorter, a
    # single segment, one-iteration segments) against the oracle, on Gaussian
    # inputs
    w = custom_workload("gram", GRAM_SHAPES, "bf16", "bf16", g_std=1.0)
    Gs = [host_tensor(w, i, GRAD, seed=7) for i in range(w.count)]
    say(f"case Gram space restart {restart} ns_steps {ns_steps}")
    outs = orth_gpu([g.cuda() for g in Gs], ns_steps=ns_steps, algo="gram_space", restart=restart)
    for i, g in enumerate(Gs):
        e = rel(f64(outs[i]), oracle.newton_schulz(f64(g), ns_steps, A, B, C, EPS))
        assert e < TOL["bf16"], (GRAM_SHAPES[i], e)


def _spectrum_input(m, n, sv, seed):
    r = np.random.default_rng(seed)
    u, _ = np.linalg.qr(r.standard_normal((m, m)))
    v, _ = np.linalg.qr(r.standard_normal((n, m)))
    return torch.from_numpy(((u * sv) @ v.T).astype(np.float32)).to(torch.bfloat16)


def test_gram_space_ill_conditioned_inputs():
    # Singular values 1 / (1 + i) and exp(-8 i / m): the Gram space squares the
    # condition number, so in bf16 it resolves small singular values far worse
    # than the short side; restarting every 3 iterations keeps its error within
    # 2x of the short side's (which itself exceeds the Gaussian-input bound on
    # such inputs), while a single 5-iteration segment is several times worse.
    m, n = 512, 1792
    cases = {"power": 1.0 / (1.0 + np.arange(m)), "exp": np.exp(-8.0 * np.arange(m) / m)}
    for name, sv in cases.items():
        x = _spectrum_input(m, n, sv, seed=12)
        ref = oracle.newton_schulz(f64(x), 5, A, B, C, EPS)
        err = {}
        for algo, restart in (("short_side", 0), ("gram_space", 3), ("gram_space", 5)):
            o = orth_gpu([x.cuda()], algo=algo, restart=restart)[0]
            err[(algo, restart)] = rel(f64(o), ref)
        say(f"case ill-conditioned {name} {m}x{n}: " + ", ".join(f"{k} {v:.3e}" for k, v in err.items()))
        short, gram3, gram5 = err[("short_side", 0)], err[("gram_space", 3)], err[("gram_space", 5)]
        assert gram3 < 2 * short
        assert gram5 > 3 * gram3


def test_gram_space_growth_bound_falls_back():
    # Beyond |a|^gram_restart = 2^64 a call runs Gram-space buckets on the short
    # side: the same products as a short-side plan, so the same bits.  Below it
    # the two forms differ (rounding), which shows the Gram space ran.  Both
    # shapes run tiled products in either plan (a 128 x n bucket with n <= 512
    # would run resident in the short-side plan, whose square rounds its b A
    # term differently).
    w = custom_workload("fallback", [(256, 768), (640, 128)], "bf16", "bf16", g_std=1.0)
    Gs = [host_tensor(w, i, GRAD, seed=6).cuda() for i in range(w.count)]
    bits = lambda t: t.view(torch.int32)
    over = math.floor(64 / math.log2(A)) + 1
    say(f"case Gram-space growth bound, restart {over}, ns_steps {over}")
    runs = [orth_gpu(Gs, ns_steps=over, algo="gram_space", restart=over),
            orth_gpu(Gs, ns_steps=over, algo="short_side")]
    for x, y in zip(*runs):
        assert torch.equal(bits(x), bits(y))
    under = [orth_gpu(Gs, ns_steps=5, algo=al) for al in ("gram_space", "short_side")]
    assert not torch.equal(under[0][0], under[1][0])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_transpose_bitwise(seed):
    # a tall matrix and its transpose run the same X in the same bucket layout,
    # with the norm taken in X's orientation: the outputs are exact transposes
    # of each other (ragged shapes included, both paths)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    for shape, dt in (((640, 256), torch.bfloat16), ((700, 300), torch.bfloat16), ((330, 130), torch.float32)):
        g = torch.randn(shape, device="cuda", generator=gen).to(dt)
        say(f"case transpose ns_orthogonalize_batched seed {seed} shape {shape} {dt}")
        o_tall, o_wide = orth_gpu([g, g.t().contiguous()])
        assert torch.equal(o_tall, o_wide.t())


def test_batch_invariance_and_determinism():
    w = custom_workload("inv", [(384, 896), (896, 384), (256, 256), (128, 512)], "bf16", "bf16")
    Gs = [host_tensor(w, i, GRAD, seed=9).cuda() for i in range(w.count)]
    say("case batch invariance ns_orthogonalize_batched")
    full = orth_gpu(Gs)
    again = orth_gpu(Gs)
    for a_, b_ in zip(full, again):
        assert torch.equal(a_, b_)
    alone = orth_gpu([Gs[1]])[0]
    assert torch.equal(alone, full[1])
    reordered = orth_gpu([Gs[3], Gs[1], Gs[0]])
    assert torch.equal(reordered[1], full[1]) and torch.equal(reordered[0], full[3])


def test_two_steps_and_checkpoint_restart():
    w = get_workload("bf16_small_batch_96")
    say("case two steps vs checkpoint restart")
    G, M, W = make_inputs(w, "cuda", seed=1)
    M2, W2 = [x.clone() for x in M], [x.clone() for x in W]
    host = [(f64(g), f64(m), f64(x)) for g, m, x in zip(G, M, W)]
    plan = d.plan_for(G, [x.dtype for x in W])
    ws = d.workspace_for(plan)
    d.muon_step_batched(plan, G, M, W, workspace=ws)
    d.muon_step_batched(plan, G, M, W, workspace=ws)
    d.muon_step_batched(plan, G, M2, W2, workspace=ws)
    torch.cuda.synchronize()
    Mc = [x.cpu().clone() for x in M2]
    Wc = [x.cpu().clone() for x in W2]
    M3, W3 = [x.cuda() for x in Mc], [x.cuda() for x in Wc]
    d.muon_step_batched(plan, G, M3, W3, workspace=d.workspace_for(plan))
    torch.cuda.synchronize()
    for i in range(w.count):
        assert torch.equal(M[i], M3[i]) and torch.equal(W[i], W3[i])
    # two oracle steps on a few matrices (bf16 parameter rounded between steps)
    for i in (0, 40, 80):
        g, m, x = host[i]
        r1 = oracle.muon_step(g, m, x, lr=LR, beta=BETA, eps=EPS)
        x1 = oracle.round_to_bf16(r1["W_new"])
        r2 = oracle.muon_step(g, oracle.round_to_f32(r1["M_new"]), x1, lr=LR, beta=BETA, eps=EPS)
        assert rel(f64(M[i]), r2["M_new"]) < 1e-6
        spec = w.matrices[i]
        check_param(f64(W[i]), x1, r2, "bf16", "bf16", spec.rows, spec.cols)


# ---- full size: the benchmark's owner share and the two full Qwen projection sets -----
# One oracle sample per distinct (rows, cols), i.e. per shape and orientation.

FULL_SETS = ["llama3.1-8b_owner_1of8", "qwen2.5-1.5b_proj", "qwen2.5-7b_proj"]


def _samples(w):
    picks = {}
    for i, s in enumerate(w.matrices):
        picks.setdefault((s.rows, s.cols), i)
    return sorted(picks.values())


@pytest.mark.parametrize("wname", FULL_SETS)
def test_full_size_step_sampled(wname):
    w = get_workload(wname)
    say(f"case {wname} full muon_step_batched ({w.count} matrices, {w.elements()} elements)")
    G, M, W = make_inputs(w, "cuda", seed=0)
    sample = _samples(w)
    host = {i: (f64(G[i]), f64(M[i]), f64(W[i])) for i in sample}
    M0 = [x.clone() for x in M]
    plan = d.plan_for(G, [x.dtype for x in W])
    ws = d.workspace_for(plan)
    d.muon_step_batched(plan, G, M, W, workspace=ws)
    torch.cuda.synchronize()
    refs = {}
    for i in sample:
        spec = w.matrices[i]
        say(f"  oracle sample {i} {spec.name} {spec.rows}x{spec.cols}")
        refs[i] = ref = oracle.muon_step(*host[i], lr=LR, beta=BETA, eps=EPS)
        assert rel(f64(M[i]), ref["M_new"]) < 1e-6
        check_param(f64(W[i]), host[i][2], ref, "bf16", "bf16", spec.rows, spec.cols)
    del W, ws
    # The same step through the same path on the same G and M, with zero fp32
    # parameters: W' = -lr s O exposes the step's own O, held to 2e-2 per sample
    # (the bf16 W' bound above is dominated by the parameter's rounding).
    say(f"case {wname} full muon_step_batched, fp32 zero params")
    Z = [torch.zeros(x.shape, dtype=torch.float32, device="cuda") for x in G]
    plan = d.plan_for(G, [torch.float32] * len(G))
    ws = d.workspace_for(plan)
    d.muon_step_batched(plan, G, M0, Z, workspace=ws)
    torch.cuda.synchronize()
    for i in sample:
        spec = w.matrices[i]
        assert torch.equal(M0[i], M[i])
        O = -f64(Z[i]) / (LR * oracle.update_scale(spec.rows, spec.cols))
        e = rel(O, refs[i]["O"])
        say(f"  O through the step, sample {i} {spec.rows}x{spec.cols}: rel err {e:.3e}")
        assert e < TOL["bf16"]
    del G, M, M0, Z, ws
    torch.cuda.empty_cache()


FULL_ORTH = [(wn, "auto") for wn in FULL_SETS] + [("llama3.1-8b_owner_1of8", "short_side")]


@pytest.mark.parametrize("wname,algo", FULL_ORTH)
def test_full_size_orthogonalize_sampled(wname, algo):
    w = get_workload(wname)
    say(f"case {wname} full ns_orthogonalize_batched bf16 in, fp32 out, {algo}")
    G, _, _ = make_inputs(w, "cuda", seed=2)
    outs = orth_gpu(G, algo=algo)
    for i in _samples(w):
        spec = w.matrices[i]
        say(f"  oracle sample {i} {spec.name} {spec.rows}x{spec.cols}")
        ref = oracle.newton_schulz(f64(G[i]), 5, A, B, C, EPS)
        e = rel(f64(outs[i]), ref)
        say(f"    rel err {e:.3e}")
        assert e < TOL["bf16"]
    del G, outs
    torch.cuda.empty_cache()


# ---- beyond 2^31 elements in one matrix ---------------------------------------------
#
# A matrix that is zero except for a few dense blocks in distinct rows and
# columns is, up to a permutation of rows and columns, block diagonal; the
# Newton-Schulz iteration keeps that structure (every product of block-diagonal
# matrices is block diagonal, p(0) = 0) and commutes with the permutation, and
# the Frobenius normalisation sees only the blocks.  So the full-size output is
# the oracle's output on the small block-diagonal matrix of the same blocks,
# scattered back, and exactly zero everywhere else.  Two matrices of 16500 x
# 131200 (2.16e9 elements, a wide and a tall one) put blocks past element 2^31.
BIG_BLOCKS = [(0, 0, 64, 200), (8000, 70000, 100, 150), (16400, 130900, 50, 300)]  # row, col, rows, cols


def test_beyond_2_31_elements_block_structure():
    r, c = 16500, 131200
    rng = np.random.default_rng(31)
    blocks = [torch.from_numpy(rng.standard_normal((br, bc)).astype(np.float32)).to(torch.bfloat16)
              for (_, _, br, bc) in BIG_BLOCKS]
    # the small block-diagonal matrix the oracle sees
    sr, sc = sum(b[2] for b in BIG_BLOCKS), sum(b[3] for b in BIG_BLOCKS)
    small = np.zeros((sr, sc))
    pos = []
    i0 = j0 = 0
    for blk, (_, _, br, bc) in zip(blocks, BIG_BLOCKS):
        small[i0:i0 + br, j0:j0 + bc] = f64(blk)
        pos.append((i0, j0))
        i0, j0 = i0 + br, j0 + bc
    ref = oracle.newton_schulz(small, 5, A, B, C, EPS)
    say(f"case {r}x{c} and {c}x{r} bf16 ({r * c} elements each) muon_step_batched, fp32 zero params")
    G = [torch.zeros(r, c, dtype=torch.bfloat16, device="cuda"), torch.zeros(c, r, dtype=torch.bfloat16, device="cuda")]
    for blk, (br0, bc0, br, bc) in zip(blocks, BIG_BLOCKS):
        G[0][br0:br0 + br, bc0:bc0 + bc] = blk.cuda()
        G[1][bc0:bc0 + bc, br0:br0 + br] = blk.t().cuda()  # the tall matrix holds the transposed blocks
    M = [torch.zeros(x.shape, device="cuda") for x in G]
    W = [torch.zeros(x.shape, device="cuda") for x in G]
    plan = d.plan_for(G, [torch.float32] * 2)
    ws = d.workspace_for(plan)
    d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(M[k], G[k].float())  # M' = 0.95 * 0 + G, exactly
        s_upd = oracle.update_scale(*W[k].shape)
        got = np.zeros((sr, sc))
        for (br0, bc0, br, bc), (i0, j0) in zip(BIG_BLOCKS, pos):
            if k == 0:
                got[i0:i0 + br, j0:j0 + bc] = f64(W[0][br0:br0 + br, bc0:bc0 + bc]) / (-LR * s_upd)
            else:
                got[i0:i0 + br, j0:j0 + bc] = f64(W[1][bc0:bc0 + bc, br0:br0 + br]).T / (-LR * s_upd)
        # every nonzero of W' lies in a block
        assert int(torch.count_nonzero(W[k])) == int(np.count_nonzero(got))
        e = rel(got, ref)
        say(f"  {'wide' if k == 0 else 'tall'}: rel err {e:.3e}")
        assert e < TOL["bf16"]
    del G, M, W, ws
    torch.cuda.empty_cache()
