"""Pins of the fp64 oracle against what the mathematics fixes (CPU only).

None of these re-types the oracle's matrix arithmetic: each compares it with a
different computation -- LAPACK's SVD, exact rational evaluation of the scalar
polynomial, closed forms of special inputs, or invariances that a dropped term,
a wrong sign, a wrong coefficient or a transposed operand would break.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

from oracle import (NS_COEFFS, apply_update, frobenius_normalize, momentum, muon_step,
                    newton_schulz, ns_cost, round_to_bf16, update_scale)

A_, B_, C_ = NS_COEFFS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def p_scalar(s, steps):
    """Scalar quintic, applied ``steps`` times (the closed form of NS on one
    singular value)."""
    for _ in range(steps):
        s = A_ * s + B_ * s ** 3 + C_ * s ** 5
    return s


def svd_closed_form(G, steps, eps):
    """NS(G) = U p^steps(S / (||G||_F + eps)) V^T, from LAPACK's thin SVD."""
    U, S, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    fro = math.sqrt(float(np.sum(S * S)))
    return (U * p_scalar(S / (fro + eps), steps)) @ Vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def rng(seed=0):
    return np.random.default_rng(seed)


# --- P1: SVD closed form -------------------------------------------------------

@pytest.mark.parametrize("shape", [(8, 12), (12, 8), (16, 16), (5, 9), (9, 5), (1, 7), (7, 1)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_svd_closed_form(shape, steps):
    G = rng(1).standard_normal(shape)
    got = newton_schulz(G, steps, eps=1e-7)
    want = svd_closed_form(G, steps, eps=1e-7)
    assert got.shape == G.shape
    assert rel(got, want) < 1e-12


def test_svd_closed_form_other_coefficients():
    # a different (cubic) polynomial: the oracle must use the coefficients it is given
    G = rng(2).standard_normal((6, 10))
    a, b, c = 1.5, -0.5, 0.0
    got = newton_schulz(G, 3, a, b, c, eps=0.0)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = S / math.sqrt(float(np.sum(S * S)))
    for _ in range(3):
        s = a * s + b * s ** 3 + c * s ** 5
    assert rel(got, (U * s) @ Vt) < 1e-12


# --- P2: diagonal inputs, against exact rational values ---------------------------

def load_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "quintic_exact.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, k, v = line.split()
            vals[(s, int(k))] = float(v)
    return vals


def test_golden_matches_exact_rational():
    # the stored file is what exact rational arithmetic gives (regenerated here)
    a, b, c = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")
    for (s, k), v in load_golden().items():
        x = Fraction(s)
        for _ in range(k):
            x = a * x + b * x ** 3 + c * x ** 5
        assert float(x) == v
    assert a + b + c == Fraction("0.701")


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_diagonal_single_entry(steps):
    # a 1-entry diagonal normalises to exactly 1 (eps = 0): O_00 = p^k(1)
    g = load_golden()
    for r, c in [(3, 5), (5, 3), (4, 4)]:
        G = np.zeros((r, c))
        G[0, 0] = 2.5
        O = newton_schulz(G, steps, eps=0.0)
        assert abs(O[0, 0] - g[("1", steps)]) < 1e-14
        O[0, 0] = 0.0
        assert np.all(O == 0.0)


def test_diagonal_entries_golden():
    # d = (0.5, sqrt(1 - 0.25 - 0.01), 0.1) has unit norm, so with eps = 0 the
    # normalised entries 0.5 and 0.1 are tabulated points of the golden file.
    g = load_golden()
    d = np.array([0.5, math.sqrt(1.0 - 0.25 - 0.01), 0.1])
    for shape in [(3, 7), (7, 3), (3, 3)]:
        G = np.zeros(shape)
        for i, v in enumerate(d):
            G[i, i] = v
        O = newton_schulz(G, 5, eps=0.0)
        assert abs(O[0, 0] - g[("0.5", 5)]) < 1e-13
        assert abs(O[2, 2] - g[("0.1", 5)]) < 1e-13
        assert abs(O[1, 1] - p_scalar(d[1], 5)) < 1e-13
        off = O.copy()
        for i in range(3):
            off[i, i] = 0
        assert np.all(off == 0.0)


def test_diagonal_signs_and_eps():
    d = np.array([3.0, -1.0, 0.25, -0.01])
    G = np.zeros((4, 6))
    for i, v in enumerate(d):
        G[i, i] = v
    eps = 1e-3
    O = newton_schulz(G, 5, eps=eps)
    nrm = float(np.sqrt(np.sum(d * d)))
    for i, v in enumerate(d):
        assert abs(O[i, i] - math.copysign(p_scalar(abs(v) / (nrm + eps), 5), v)) < 1e-13


# --- P3 rank-1, P8 special cases ----------------------------------------------

def test_rank_one():
    r = rng(3)
    u, v = r.standard_normal(9), r.standard_normal(13)
    G = np.outer(u, v)
    eps = 1e-7
    O = newton_schulz(G, 5, eps=eps)
    s = p_scalar(1.0 / (1.0 + eps / np.linalg.norm(G)), 5)
    want = s * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert rel(O, want) < 1e-12
    assert abs(s - load_golden()[("1", 5)]) < 1e-5


def test_steps_zero_is_normalisation():
    G = rng(4).standard_normal((6, 11)) * 7.0
    eps = 0.5
    O = newton_schulz(G, 0, eps=eps)
    assert rel(O, G / (math.sqrt(float((G ** 2).sum())) + eps)) < 1e-15
    X0 = frobenius_normalize(G, 0.0)
    assert abs(np.linalg.norm(X0) - 1.0) < 1e-14


def test_zero_input():
    G = np.zeros((5, 8))
    O = newton_schulz(G, 5, eps=1e-7)
    assert np.all(O == 0.0)
    M0 = np.zeros((5, 8))
    W = rng(5).standard_normal((5, 8))
    out = muon_step(G, M0, W)
    assert np.all(out["M_new"] == 0.0) and np.all(out["W_new"] == W)


@pytest.mark.parametrize("m,n", [(4, 9), (6, 6), (3, 20)])
def test_orthonormal_rows(m, n):
    Q, _ = np.linalg.qr(rng(6).standard_normal((n, m)))
    G = Q.T  # m x n with G G^T = I
    eps = 1e-7
    O = newton_schulz(G, 5, eps=eps)
    assert rel(O, p_scalar(1.0 / (math.sqrt(m) + eps), 5) * G) < 1e-12
    Ot = newton_schulz(G.T, 5, eps=eps)
    assert rel(Ot, p_scalar(1.0 / (math.sqrt(m) + eps), 5) * G.T) < 1e-12


# --- P4-P6 invariances ------------------------------------------------------------

@pytest.mark.parametrize("shape", [(7, 7), (6, 10), (10, 6)])
def test_transpose_consistency(shape):
    G = rng(7).standard_normal(shape)
    assert rel(newton_schulz(G.T, 5), newton_schulz(G, 5).T) < 1e-12


def test_scaling_and_sign():
    G = rng(8).standard_normal((6, 9))
    base = newton_schulz(G, 5, eps=0.0)
    for alpha in (1e-3, 0.37, 5.0, 1e4):
        assert rel(newton_schulz(alpha * G, 5, eps=0.0), base) < 1e-12
    assert np.array_equal(newton_schulz(-G, 5, eps=0.0), -base)


def test_orthogonal_equivariance():
    r = rng(9)
    G = r.standard_normal((5, 8))
    U, _ = np.linalg.qr(r.standard_normal((5, 5)))
    V, _ = np.linalg.qr(r.standard_normal((8, 8)))
    assert rel(newton_schulz(U @ G @ V, 5), U @ newton_schulz(G, 5) @ V) < 1e-12


# --- P7 invariant band ------------------------------------------------------------

def band_edges():
    """Critical points of p: roots of a + 3 b s^2 + 5 c s^4 = 0 (quadratic in s^2)."""
    qa, qb, qc = 5 * C_, 3 * B_, A_
    disc = math.sqrt(qb * qb - 4 * qa * qc)
    s1 = math.sqrt((-qb - disc) / (2 * qa))
    s2 = math.sqrt((-qb + disc) / (2 * qa))
    return s1, s2, p_scalar(s1, 1), p_scalar(s2, 1)


def test_band_edges_values():
    s1, s2, pmax, pmin = band_edges()
    assert abs(s1 - 0.55452879) < 1e-7 and abs(s2 - 1.05013608) < 1e-7
    assert abs(pmax - 1.2023686) < 1e-6 and abs(pmin - 0.6818310) < 1e-6
    grid = np.linspace(pmin, pmax, 20001)
    img = p_scalar(grid, 1)
    assert img.min() >= pmin - 1e-12 and img.max() <= pmax + 1e-12


@pytest.mark.parametrize("lo,upper", [(2e-3, None), (1e-2, 1.13436)])
def test_band_controlled_spectrum(lo, upper):
    _, _, pmax, pmin = band_edges()
    hi = pmax if upper is None else upper
    r = rng(10)
    m, n = 12, 20
    U, _ = np.linalg.qr(r.standard_normal((m, m)))
    V, _ = np.linalg.qr(r.standard_normal((n, m)))
    for trial in range(5):
        s = np.exp(r.uniform(math.log(lo), 0.0, size=m))
        s[0] = 1.0
        s = s / math.sqrt(float(np.sum(s * s)))
        s = np.maximum(s, lo)
        G = (U * s) @ V.T
        shat = np.linalg.svd(G, compute_uv=False) / np.linalg.norm(G)
        if shat.min() < lo:
            continue
        out = np.linalg.svd(newton_schulz(G, 5, eps=0.0), compute_uv=False)
        assert out.min() >= pmin - 1e-9 and out.max() <= hi + 1e-9


# --- P9 zero padding --------------------------------------------------------------

def test_zero_padding():
    G = rng(11).standard_normal((5, 9))
    base = newton_schulz(G, 5)
    P = np.zeros((8, 16))
    P[:5, :9] = G
    out = newton_schulz(P, 5)
    assert rel(out[:5, :9], base) < 1e-13
    assert np.all(out[5:, :] == 0.0) and np.all(out[:, 9:] == 0.0)


# --- momentum, update, cost ---------------------------------------------------------

def test_momentum_geometric_series():
    # constant gradient from zero momentum: M_k = G (1 - beta^k) / (1 - beta)
    G = rng(12).standard_normal((4, 6))
    beta = 0.95
    M = np.zeros_like(G)
    for k in range(1, 8):
        M, U = momentum(G, M, beta, nesterov=True)
        geo = (1 - beta ** k) / (1 - beta)
        assert rel(M, geo * G) < 1e-14
        assert rel(U, (1 + beta * geo) * G) < 1e-14
        M_plain, U_plain = momentum(G, M, beta, nesterov=False)  # plain form: U = M'
        assert np.array_equal(U_plain, M_plain)


def test_momentum_forms_agree_on_direction_from_zero():
    # from M0 = 0 the damped (EMA) form's look-ahead (1-beta)(1+beta) G is parallel
    # to the accumulate form's (1+beta) G: the orthogonalised direction is the same
    G = rng(13).standard_normal((5, 7))
    beta = 0.9
    _, U = momentum(G, np.zeros_like(G), beta)
    assert rel(U, (1 + beta) * G) < 1e-15
    ema_U = (1 - beta) * G + beta * (beta * 0.0 + (1 - beta) * G)
    assert rel(newton_schulz(U, 5, eps=0.0), newton_schulz(ema_U, 5, eps=0.0)) < 1e-12


def test_update_scale_ratio():
    G = rng(14).standard_normal((24, 6))  # tall: rows/cols = 4 -> scale 2
    assert update_scale(24, 6) == 2.0 and update_scale(6, 24) == 1.0 and update_scale(5, 5) == 1.0
    Z = np.zeros_like(G)
    tall = muon_step(G, Z, Z, lr=0.1, beta=0.0)
    wide = muon_step(G.T, Z.T, Z.T, lr=0.1, beta=0.0)
    ratio = np.linalg.norm(tall["W_new"]) / np.linalg.norm(wide["W_new"])
    assert abs(ratio - 2.0) < 1e-12
    assert rel(tall["W_new"], -0.1 * 2.0 * newton_schulz(G, 5)) < 1e-12


def test_weight_decay_and_lr():
    W = rng(15).standard_normal((3, 4))
    O = rng(16).standard_normal((3, 4))
    got = apply_update(W, O, lr=0.5, scale=1.0, weight_decay=0.2)
    assert rel(got, 0.9 * W - 0.5 * O) < 1e-15


def test_ns_cost_values():
    assert ns_cost(4096, 14336) == 4 * 4096 ** 2 * 14336 + 2 * 4096 ** 3
    assert ns_cost(14336, 4096) == ns_cost(4096, 14336)
    assert ns_cost(128, 128) == 6 * 128 ** 3


# --- bf16 rounding ------------------------------------------------------------------

def test_bf16_rounding_ties_and_library():
    one = 1.0
    assert round_to_bf16(np.array([one + 2 ** -8]))[0] == 1.0             # tie -> even
    assert round_to_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6  # tie -> even
    assert round_to_bf16(np.array([one + 2 ** -8 + 2 ** -30]))[0] == 1.0 + 2 ** -7
    assert round_to_bf16(np.array([-3.0]))[0] == -3.0
    import torch

    x = rng(17).standard_normal(20000) * np.exp(rng(18).uniform(-20, 20, 20000))
    x = x.astype(np.float32).astype(np.float64)  # torch rounds from fp32
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x), want)


@pytest.mark.parametrize("shape", [(12, 40), (40, 12), (16, 16), (7, 9)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_gram_space_recurrence_matches_definition(shape, steps):
    # the Gram-space recurrence reaches the short-side iteration's result exactly
    # (up to fp64 rounding), and both match the SVD closed form
    rng = np.random.default_rng(sum(shape) + steps)
    G = rng.standard_normal(shape)
    ref = oracle.newton_schulz(G, steps)
    got = oracle.gram_newton_schulz(G, steps)
    assert np.linalg.norm(got - ref) <= 1e-12 * max(np.linalg.norm(ref), 1.0)
    u, sv, vt = np.linalg.svd(G, full_matrices=False)
    x = sv / (np.linalg.norm(G) + 1e-7)
    for _ in range(steps):
        x = A_ * x + B_ * x ** 3 + C_ * x ** 5
    assert np.linalg.norm(got - (u * x) @ vt) <= 1e-11 * max(np.linalg.norm(got), 1.0)


def test_non_finite_inputs_propagate():
    """Reading: non-finite gradients are not masked.  Momentum is elementwise,
    so only the planted entry of M' is non-finite; the norm is NaN or Inf, so
    X is NaN in at least one entry, the Gram product spreads it over a row and
    a column and the square over everything: O and W' are NaN everywhere."""
    rng = np.random.default_rng(11)
    for val, shape in ((np.nan, (6, 10)), (np.inf, (10, 6)), (-np.inf, (7, 7))):
        G = rng.standard_normal(shape)
        M = rng.standard_normal(shape)
        W = rng.standard_normal(shape)
        G[2, 3] = val
        with np.errstate(invalid="ignore"):  # Inf / Inf in the normalisation
            out = oracle.muon_step(G, M, W)
        bad = ~np.isfinite(out["M_new"])
        assert bad[2, 3] and bad.sum() == 1
        if np.isnan(val):
            assert np.isnan(out["M_new"][2, 3])
        else:
            assert out["M_new"][2, 3] == val
        assert np.isnan(out["O"]).all() and np.isnan(out["W_new"]).all()
