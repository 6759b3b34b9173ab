"""Invariances of the Newton-Schulz map, checked on the GPU path itself
(ns_orthogonalize_batched through the C ABI), not only on the oracle.

The method keeps Muon's update semantics: the output depends on the input's
direction only, and it commutes with orthogonal changes of basis on either
side (DMuon explainer on gist.science, section 1 on the orthogonalisation,
sections 3 and 5 on unchanged semantics).  Here:

* positive scaling.  The library folds the normalisation 1 / (||U||_F + eps)
  into the epilogues of the first products, after an unnormalised fp32
  accumulation, so the dynamic range it handles is the input's own.  With
  eps = 0 and alpha a power of two, alpha G is exact in bf16 and fp32, and
  every later quantity -- the squares and their sums, the norm, its
  reciprocal, the first Gram product and its scale, the first B X product --
  scales by an exact power of two, so the outputs must be bitwise equal as
  long as no square, product, partial sum or accumulator leaves the normal
  fp32 range: every nonzero |u_i u_j| >= 2^-126 (1.2e-38) and
  ||U||_F^2 < 3.4e38.  On these N(0, 1e-3^2) inputs (a few million elements,
  the smallest nonzero |u| near 4e-10) that is alpha from 2^-27 to 2^60
  (at 2^60, ||U||_F^2 reaches 4e36 on the 1024 x 3072 matrix), for both forms
  of the recurrence and both paths.  Outside that range squares of the
  smallest entries turn subnormal (below) or the norm overflows (above).
  Non-power-of-two factors (1e8, 3e-8) change the input's bf16 rounding, so
  they are held to the oracle at the path's tolerance.
* sign: NS(-G) = -NS(G), the polynomial being odd.  On the fp32 path every
  operation rounds to nearest even, which is sign-symmetric, so the outputs
  are exact negatives bit for bit.  The bf16 path's matrix-core products are
  not sign-symmetric in their last fp32 bit (the accumulator's internal
  rounding of the dot product depends on the signs of the addends: measured
  on v_mfma_f32_32x32x16_bf16 with random operands, D(-A, B, -C) differs from
  -D(A, B, C) in some outputs), and a last-bit difference before a bf16
  rounding can flip it; there both signs are held to the oracle at 2e-2 and
  to each other at twice that.
* orthogonal equivariance NS(U G V) = U NS(G) V with random orthogonal U, V.
  On the fp32 path both sides are held to the oracle's NS(U G V) at 1e-4 and
  to each other at 2e-4 (triangle inequality).  On the bf16 path U G V is
  rounded to bf16 before the GPU sees it, which itself moves the exact
  result by d_in (measured on the oracle, fp64); the bound is
  2 * 2e-2 + d_in.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from matrix_optimizer_02_amd import dmuon_ns as d

pytestmark = pytest.mark.gpu

A, B, C = oracle.NS_COEFFS
TOL = {"bf16": 2e-2, "f32": 1e-4}
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def orth(inputs, algo="auto", eps=0.0, ns_steps=5):
    plan = d.plan_for(inputs, [torch.float32] * len(inputs), algo)
    ws = d.workspace_for(plan)
    outs = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in inputs]
    d.ns_orthogonalize_batched(plan, inputs, outs, ns_steps=ns_steps, eps=eps, workspace=ws)
    torch.cuda.synchronize()
    return outs, plan


def inputs(shapes, dt, std, seed):
    gen = torch.Generator().manual_seed(seed)
    return [(torch.randn(s, generator=gen) * std).to(TD[dt]).cuda() for s in shapes]


# bf16: a short-side bucket, a tall one, a resident one and a Gram-space one
# (padded short side 1024, n >= 3 m); fp32: the single-matrix shape and a ragged one
SCALE_SETS = {"bf16": [(300, 700), (700, 300), (128, 384), (1024, 3072)],
              "f32": [(256, 512), (130, 77)]}
POW2 = [-27, -13, -1, 1, 13, 27, 60]


@pytest.mark.parametrize("algo", ["auto", "short_side"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_scaling_by_powers_of_two_is_bitwise(dt, algo):
    G = inputs(SCALE_SETS[dt], dt, 1e-3, seed=41)
    base, plan = orth(G, algo)
    if dt == "bf16" and algo == "auto":
        assert d.ALGO_GRAM_SPACE in {plan.bucket(b).algo for b in range(plan.info()[1])}
    for i, g in enumerate(G):
        e = rel(f64(base[i]), oracle.newton_schulz(f64(g), 5, A, B, C, 0.0))
        assert e < TOL[dt], (SCALE_SETS[dt][i], e)
    for k in POW2:
        say(f"case scaling {dt} {algo} alpha = 2^{k}")
        Gs = [(g.to(torch.float64) * 2.0 ** k).to(g.dtype) for g in G]
        for g, gs in zip(G, Gs):  # the scaled input is exact
            assert torch.equal(gs.to(torch.float64), g.to(torch.float64) * 2.0 ** k)
        outs, _ = orth(Gs, algo)
        for i in range(len(G)):
            assert torch.equal(outs[i], base[i]), (k, SCALE_SETS[dt][i], rel(f64(outs[i]), f64(base[i])))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_scaling_by_other_factors_meets_the_oracle(dt):
    G = inputs(SCALE_SETS[dt], dt, 1e-3, seed=42)
    for alpha in (1e8, 3e-8):
        say(f"case scaling {dt} alpha = {alpha:g}")
        Gs = [(g.to(torch.float64) * alpha).to(g.dtype) for g in G]
        outs, _ = orth(Gs, eps=0.0)
        for i, gs in enumerate(Gs):
            e = rel(f64(outs[i]), oracle.newton_schulz(f64(gs), 5, A, B, C, 0.0))
            assert e < TOL[dt], (alpha, SCALE_SETS[dt][i], e)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sign(dt):
    G = inputs(SCALE_SETS[dt], dt, 1e-3, seed=43)
    say(f"case sign {dt}")
    pos, _ = orth(G, eps=1e-7)
    neg, _ = orth([-g for g in G], eps=1e-7)
    for i, (p, n) in enumerate(zip(pos, neg)):
        if dt == "f32":
            assert torch.equal(n, -p), SCALE_SETS[dt][i]
            continue
        ref = oracle.newton_schulz(f64(G[i]), 5, A, B, C, 1e-7)
        e_p, e_n, e_pn = rel(f64(p), ref), rel(-f64(n), ref), rel(-f64(n), f64(p))
        say(f"  {SCALE_SETS[dt][i]}: NS(G) {e_p:.2e}, -NS(-G) {e_n:.2e}, apart {e_pn:.2e}")
        assert e_p < TOL[dt] and e_n < TOL[dt] and e_pn < 2 * TOL[dt]


def _orthogonal(n, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(48, 80), (80, 48), (64, 64), (130, 300)])
def test_orthogonal_equivariance(dt, shape):
    rng = np.random.default_rng(44 + shape[0])
    m, n = shape
    U, V = _orthogonal(m, rng), _orthogonal(n, rng)
    g = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(TD[dt])
    h = torch.from_numpy(U @ f64(g) @ V).to(TD[dt])  # U G V, rounded to the input dtype
    say(f"case orthogonal equivariance {dt} {m}x{n}")
    outs, _ = orth([g.cuda(), h.cuda()], eps=1e-7)
    og, oh = f64(outs[0]), f64(outs[1])
    ref_h = oracle.newton_schulz(f64(h), 5, A, B, C, 1e-7)
    ref_g = oracle.newton_schulz(f64(g), 5, A, B, C, 1e-7)
    rotated = U @ og @ V
    d_in = rel(U @ ref_g @ V, ref_h)  # what rounding U G V to the input dtype moves, exactly
    e_h, e_g, e_eq = rel(oh, ref_h), rel(og, ref_g), rel(oh, rotated)
    say(f"  NS(UGV) {e_h:.2e}, NS(G) {e_g:.2e}, NS(UGV) vs U NS(G) V {e_eq:.2e}, input rounding {d_in:.2e}")
    assert e_h < TOL[dt] and e_g < TOL[dt]
    assert e_eq < 2 * TOL[dt] + d_in
