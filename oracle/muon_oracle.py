"""fp64 CPU oracle of the owner-side Muon step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library and
imports nothing from it.

What it computes, per matrix and independently of every other matrix, in fp64
(bf16 and fp32 inputs embed exactly in fp64):

1. momentum accumulation:  M' = beta*M + G;  U = G + beta*M' (Nesterov) or U = M'
2. short-side orientation: if rows > cols, work on U^T (so X is m x n, m <= n)
3. Frobenius normalisation: X0 = U / (||U||_F + eps)
4. ``ns_steps`` quintic Newton-Schulz iterations, dense, in the order
   A = X X^T;  B = b A + c A A;  X = a X + B X
5. O = X^T if step 2 transposed, else X
6. update: W' = W (1 - lr wd) - lr * s * O with s = sqrt(max(1, rows/cols))

Sources.  The pages say that Muon applies the Newton-Schulz iteration to the
momentum-aggregated gradient of each weight matrix, driving its singular values
towards a uniform spectrum, and that the iteration needs the product X X^T of
the full matrix on one device (DMuon explainer on gist.science, "Technische
Samenvatting" section 1 Probleemstelling).  The iteration runs in the m x m
space when m < n (same explainer, the second section 2.1, Efficiente Gram
Newton-Schulz Iteratie), and the matrix's single owner runs the iteration and
the optimizer update on the full matrix (DMuon abstract, arXiv 2611.07084
listing; explainer section 2.1 Owner-Centric Executiestrategie).  DMuon changes
neither Muon's update rule nor its semantics (explainer sections 3 and 5).

The pages print no polynomial, coefficient, momentum rule or update scale.  The
quintic coefficients (3.4445, -4.7750, 2.0315), beta = 0.95 Nesterov, lr = 0.02,
5 steps and the sqrt(max(1, rows/cols)) scale are the values the benchmark
workloads fix.  The readings taken where everything is silent (eps, the
accumulate form of Nesterov momentum, weight decay 0, no transpose of square
matrices) are listed in the design notes; each function below states its own.

Pins (tests/test_oracle_pins.py, all independent of this file's arithmetic):
SVD closed form U p^k(S) V^T via LAPACK, exact diagonal action, rank-1 and
orthonormal-row special cases, transpose consistency, positive scaling and
sign oddness, orthogonal equivariance, the polynomial's invariant band,
zero-padding invariance, momentum geometric series, update-scale ratio.
"""

from __future__ import annotations

import math

import numpy as np

# Quintic Newton-Schulz coefficients (a, b, c) of p(s) = a s + b s^3 + c s^5.
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def _f64(x) -> np.ndarray:
    """Exact fp64 copy of a numpy array or a CPU torch tensor (bf16 included)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype
        x = x.detach().to("cpu")
        import torch

        return x.to(torch.float64).numpy().copy()
    return np.array(x, dtype=np.float64, copy=True)


def momentum(G, M, beta: float, nesterov: bool = True):
    """Momentum accumulation feeding the orthogonalisation.

    The pages only say that NS acts on the momentum-aggregated gradient
    (explainer section 1) and that the owner keeps the authoritative optimizer
    state (explainer section 2.1 Owner-Centric).  Reading taken: the accumulate
    form without (1 - beta) damping, M' = beta M + G, and the Nesterov look-ahead
    U = G + beta M'; without Nesterov, U = M'.

    Returns (M', U) in fp64.
    """
    G = _f64(G)
    M = _f64(M)
    M_new = beta * M + G
    U = G + beta * M_new if nesterov else M_new
    return M_new, U


def frobenius_normalize(U, eps: float):
    """X0 = U / (||U||_F + eps), the normalisation that puts every singular
    value in [0, 1] before the iteration.  eps is added to the norm so that an
    all-zero U gives X0 = 0 (reading: the pages are silent on it)."""
    U = _f64(U)
    norm = math.sqrt(float(np.sum(U * U)))
    return U / (norm + eps)


def ns_iteration(X, a: float, b: float, c: float):
    """One quintic Newton-Schulz step on an m x n matrix X (m <= n), written as
    the three products the method names: the Gram matrix A = X X^T (the product
    the explainer's section 1 singles out), B = b A + c A A, and X' = a X + B X.
    Dense: no symmetry is exploited here."""
    A = X @ X.T
    B = b * A + c * (A @ A)
    return a * X + B @ X


def newton_schulz(G, steps: int, a: float = NS_COEFFS[0], b: float = NS_COEFFS[1],
                  c: float = NS_COEFFS[2], eps: float = 1e-7):
    """Orthogonalise G: normalise, run ``steps`` iterations on the short side,
    return O in G's own orientation (fp64).

    Short side: the iteration works on the m x m Gram space with m = min(rows,
    cols) (explainer, second section 2.1).  A tall G (rows > cols) is
    transposed before and after; a square G is not transposed.
    """
    X = _f64(G)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a 2-D matrix")
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T.copy()
    X = frobenius_normalize(X, eps)
    for _ in range(int(steps)):
        X = ns_iteration(X, a, b, c)
    return X.T.copy() if transposed else X


def gram_newton_schulz(G, steps: int, a: float = NS_COEFFS[0], b: float = NS_COEFFS[1],
                       c: float = NS_COEFFS[2], eps: float = 1e-7):
    """The same map as ``newton_schulz``, run as the m x m Gram-space recurrence
    (explainer, second section 2.1: the iteration moves into the Gram space of
    the short side, lowering its cost from order m^2 n to order m^3).

    Every iterate of the short-side recurrence is X_k = P_k X_0 with P_0 = I.
    Writing A_k = X_k X_k^T = P_k A_0 P_k^T and Q_k = a I + b A_k + c A_k A_k,
    the step X_{k+1} = Q_k X_k becomes P_{k+1} = Q_k P_k and
    A_{k+1} = Q_k A_k Q_k^T; the result is O = P_steps X_0.  Dense fp64, no
    symmetry tricks; a tall G is transposed before and after, as there.
    """
    X = _f64(G)
    if X.ndim != 2:
        raise ValueError("gram_newton_schulz expects a 2-D matrix")
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T.copy()
    X0 = frobenius_normalize(X, eps)
    m = X0.shape[0]
    A = X0 @ X0.T
    P = np.eye(m)
    for _ in range(int(steps)):
        Q = a * np.eye(m) + b * A + c * (A @ A)
        P = Q @ P
        A = Q @ A @ Q.T
    O = P @ X0
    return O.T.copy() if transposed else O


def update_scale(rows: int, cols: int) -> float:
    """Per-matrix update scale s = sqrt(max(1, rows / cols)) of the stored
    (out x in) parameter: tall matrices get s > 1, wide and square ones s = 1."""
    return math.sqrt(max(1.0, rows / cols))


def apply_update(W, O, lr: float, scale: float, weight_decay: float = 0.0):
    """W' = W (1 - lr wd) - lr s O in fp64 (decoupled weight decay; 0 in every
    workload, the pages being silent on it)."""
    W = _f64(W)
    return W * (1.0 - lr * weight_decay) - lr * scale * _f64(O)


def muon_step(G, M, W, *, lr: float = 0.02, beta: float = 0.95, nesterov: bool = True,
              ns_steps: int = 5, a: float = NS_COEFFS[0], b: float = NS_COEFFS[1],
              c: float = NS_COEFFS[2], eps: float = 1e-7, weight_decay: float = 0.0):
    """One owner-side Muon step on one matrix: momentum, normalisation, NS on
    the short side, update.  The owner runs NS and the update once per matrix
    on the full matrix (DMuon abstract; explainer section 2.1 Owner-Centric).

    Returns a dict of fp64 arrays: M_new (r x c), O (r x c), W_new (r x c), and
    the scalar ``scale`` used.
    """
    M_new, U = momentum(G, M, beta, nesterov)
    O = newton_schulz(U, ns_steps, a, b, c, eps)
    r, cdim = U.shape
    s = update_scale(r, cdim)
    W_new = apply_update(W, O, lr, s, weight_decay)
    return {"M_new": M_new, "O": O, "W_new": W_new, "scale": s}


def ns_cost(m: int, n: int) -> int:
    """Dense-equivalent cost of one NS iteration on an m x n (m <= n) matrix,
    4 m^2 n + 2 m^3: X X^T (2 m^2 n), A A (2 m^3) and B X (2 m^2 n).  Exact
    integer.  Used to order work by computational cost (DMuon abstract:
    owners are balanced by computational cost)."""
    m, n = int(m), int(n)
    if m > n:
        m, n = n, m
    return 4 * m * m * n + 2 * m * m * m


def round_to_f32(x) -> np.ndarray:
    """Round fp64 to the nearest fp32 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    bf16 keeps 8 significant bits: a value with frexp exponent e (|v| in
    [2**(e-1), 2**e)) is rounded to a multiple of 2**(e-8); below the normal
    range the spacing stays 2**-133.  ``np.rint`` rounds half to even.  The
    division by a power of two is exact.  NaN/Inf and zeros pass through;
    values beyond bf16's largest finite value are not handled.
    """
    x = np.asarray(x, dtype=np.float64)
    _, exp = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(exp - 8, -133))
    with np.errstate(invalid="ignore"):
        out = np.rint(x / q) * q
    return np.where(np.isfinite(x), out, x)
