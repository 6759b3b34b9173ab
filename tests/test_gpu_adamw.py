"""GPU parity of the AdamW companion step (through the C ABI) against the fp64
oracle, on seeded inputs; each step is checked from the state the GPU held
before it.

Bounds, element by element, derived from the arithmetic:
  * moments m', v' (fp32, a handful of fp32 operations from fp32 inputs):
        |x_gpu - x_ref| <= 8 u32 (|beta x| + |(1 - beta) y|),  u32 = 2^-24
  * parameter p': the device computes p' in fp32 and rounds once to the
    parameter dtype, so
        |p_gpu - p_ref| <= 0.5 (1 + 2^-8) ulp(p_ref) + delta,
        delta = 16 u32 (|p| + lr |u|) + lr 1e-5 |u|
    where u = m_hat / (sqrt(v_hat) + eps) is the oracle's step direction
    (the 1e-5 covers the fp32 division, square root and bias corrections).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from matrix_optimizer_02_amd import dmuon_ns as d

pytestmark = pytest.mark.gpu

H = dict(oracle.ADAMW_DEFAULTS)
U32 = 2.0 ** -24


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def ulp(x, dtype):
    bits = 8 if dtype == torch.bfloat16 else 24
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - bits, -126 - bits + 1))


def make_state(n, pdt, gdt, rng, step):
    p = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 0.02).to(pdt).cuda()
    g = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 1e-3).to(gdt).cuda()
    if step == 1:
        m = torch.zeros(n, dtype=torch.float32, device="cuda")
        v = torch.zeros(n, dtype=torch.float32, device="cuda")
    else:
        m = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 1e-4).cuda()
        v = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32) ** 2).cuda()
    return p, g, m, v


def within(x, ref, bound, what, g0, s0):
    err = np.abs(x - ref)
    if not np.all(err <= bound):
        i = int(np.argmax(err / np.maximum(bound, 1e-300)))
        raise AssertionError(f"{what}: element {i} of {x.size}: gpu {x[i]!r} ref {ref[i]!r} err {err[i]:.3e} "
                             f"bound {bound[i]:.3e}; g {g0[i]!r} state {s0[i]!r}")


def check(tensors, before, step):
    for (p, g, m, v), (p0, g0, m0, v0) in zip(tensors, before):
        pr, mr, vr = oracle.adamw_step(p0, g0, m0, v0, step, **H)
        b1, b2, lr, eps = H["beta1"], H["beta2"], H["lr"], H["eps"]
        within(f64(m), mr, 8 * U32 * (np.abs(b1 * m0) + np.abs((1 - b1) * g0)) + 1e-30, "m", g0, m0)
        within(f64(v), vr, 8 * U32 * (np.abs(b2 * v0) + np.abs((1 - b2) * g0 * g0)) + 1e-38, "v", g0, v0)
        u = (mr / (1 - b1 ** step)) / (np.sqrt(vr / (1 - b2 ** step)) + eps)
        delta = 16 * U32 * (np.abs(p0) + lr * np.abs(u)) + lr * 1e-5 * np.abs(u)
        bound = 0.5 * (1 + 2.0 ** -8) * ulp(pr, p.dtype) + delta
        within(f64(p), pr, bound, "p", g0, p0)


CASES = [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
         (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)]
LENGTHS = [1, 7, 8, 9, 2047, 2048, 2049, 3 * 4096 + 5, 100003]


@pytest.mark.parametrize("pdt,gdt", CASES)
def test_adamw_parity_three_steps(pdt, gdt):
    rng = np.random.default_rng(21)
    say(f"case adamw {pdt} params {gdt} grads, lengths {LENGTHS}")
    tensors = [make_state(n, pdt, gdt, rng, step=1) for n in LENGTHS]
    for step in (1, 2, 3):
        before = [tuple(f64(x) for x in t) for t in tensors]
        P, G, M, V = (list(x) for x in zip(*tensors))
        d.adamw_step_batched(P, G, M, V, step=step, lr=H["lr"], betas=(H["beta1"], H["beta2"]),
                             eps=H["eps"], weight_decay=H["weight_decay"])
        torch.cuda.synchronize()
        check(tensors, before, step)
        # a new gradient for the next step
        for t in tensors:
            t[1].copy_(torch.from_numpy(rng.standard_normal(t[1].numel()).astype(np.float32) * 1e-3))


def test_adamw_many_tensors_and_empty_ones():
    # more tensors than one launch carries, mixed dtypes, empty tensors skipped,
    # a later step with non-zero moments
    rng = np.random.default_rng(22)
    lengths = [int(x) for x in rng.integers(0, 5000, size=150)] + [0, 0, 70001]
    say(f"case adamw {len(lengths)} tensors (several launches), step 10")
    tensors = [make_state(n, CASES[i % 4][0], CASES[i % 4][1], rng, step=10) for i, n in enumerate(lengths)]
    before = [tuple(f64(x) for x in t) for t in tensors]
    P, G, M, V = (list(x) for x in zip(*tensors))
    d.adamw_step_batched(P, G, M, V, step=10)
    torch.cuda.synchronize()
    check(tensors, before, 10)


def test_adamw_zero_gradient_is_decay_only():
    n = 4099
    p = (torch.arange(n, dtype=torch.float32, device="cuda") - 2000.0) * 1e-3
    g = torch.zeros(n, device="cuda")
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    p0 = f64(p)
    say("case adamw zero gradient")
    d.adamw_step_batched([p], [g], [m], [v], step=1)
    torch.cuda.synchronize()
    expect = p0 * np.float64(np.float32(1 - H["lr"] * H["weight_decay"]))
    assert np.all(np.abs(f64(p) - expect) <= U32 * np.abs(expect))
    assert not m.any() and not v.any()
