"""The measurement kernels the benchmark reports its ceilings with: the copy
moves the bytes it is given, the matrix-core burn leaves finite sums, and the
clock sampler's readings advance monotonically at a plausible shader clock.
Argument checks are refused before anything is enqueued."""

import pytest
import torch

from matrix_optimizer_02_amd import dmuon_ns as d

pytestmark = pytest.mark.gpu


def test_copy_is_exact():
    src = torch.randn(3 * 1024 * 1024 + 4, device="cuda")  # not a multiple of the grid's stride
    dst = torch.empty_like(src)
    d.diag_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_copy_refuses_bad_arguments():
    src = torch.zeros(1024, device="cuda")
    with pytest.raises(ValueError):
        d.diag_copy(torch.zeros(512, device="cuda"), src)
    with pytest.raises(d.DMuonError):
        d.diag_copy(src, src)  # overlapping


def test_mfma_burn_is_finite():
    out = torch.zeros(8 * 512, device="cuda")
    flops = d.diag_mfma(out, 8, 64)
    torch.cuda.synchronize()
    # blocks x waves x iterations x eight accumulators x one 32 x 32 x 16 MFMA
    assert flops == 8 * 8 * 64 * 8 * (2 * 32 * 32 * 16)
    assert torch.isfinite(out).all() and (out != 0).any()


def test_clock_sampler_is_paced_by_the_wall_clock():
    samples, interval = 64, 10000  # 100 us apart, 6.3 ms in all
    buf = torch.zeros(2 * samples, dtype=torch.int64, device="cuda")
    d.diag_clock(buf, samples, interval)
    torch.cuda.synchronize()
    v = buf.view(samples, 2).cpu()
    # sample k waits until k intervals after the start (a few ticks before sample 0)
    since = v[:, 1] - v[0, 1]
    due = torch.arange(samples, dtype=torch.int64) * interval
    assert (since >= due - 100).all() and (since < due + 20 * interval).all()
    assert (v[1:, 0] > v[:-1, 0]).all()
    mhz = float((v[-1, 0] - v[0, 0]) / (v[-1, 1] - v[0, 1]) * 100.0)
    assert 100.0 < mhz < 3000.0, mhz
    with pytest.raises(d.DMuonError):
        d.diag_clock(buf, 1, interval)


@pytest.mark.parametrize("kind", ["prep", "apply", "adamw"])
def test_mix_kernels_compute_their_update(kind):
    n = 4 * 1000 + 1024 * 4  # not a multiple of a block's share
    gen = torch.Generator().manual_seed(7)
    a = torch.randn(n, generator=gen).to(torch.bfloat16).cuda()
    b = torch.randn(n, generator=gen).to(torch.float32 if kind == "prep" else torch.bfloat16).cuda()
    c = (torch.zeros(n, dtype=torch.bfloat16).cuda() if kind == "prep" else
         torch.rand(2 * n, generator=gen).cuda() if kind == "adamw" else None)
    a0, b0, c0 = a.float().cpu(), b.float().cpu(), None if c is None else c.float().cpu()
    nbytes = d.diag_mix(kind, a, b, c)
    torch.cuda.synchronize()
    assert nbytes == d.MIX_KINDS[kind][1] * n
    if kind == "prep":
        m = 0.95 * b0 + a0
        assert torch.allclose(b.cpu(), m, rtol=1e-6, atol=1e-6)
        assert torch.allclose(c.float().cpu(), 0.95 * m + a0, rtol=1e-2, atol=1e-2)
    elif kind == "apply":
        assert torch.allclose(b.float().cpu(), b0 - 1e-3 * a0, rtol=1e-2, atol=1e-2)
    else:
        m = 0.9 * c0[:n] + 0.1 * b0
        v = 0.999 * c0[n:] + 1e-3 * b0 * b0
        assert torch.allclose(c.cpu()[:n], m, rtol=1e-5, atol=1e-6)
        assert torch.allclose(c.cpu()[n:], v, rtol=1e-5, atol=1e-6)
        assert torch.allclose(a.float().cpu(), a0 - 1e-4 * m / (v.sqrt() + 1e-8), rtol=1e-2, atol=1e-2)


def test_mix_refuses_overlap():
    a = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(4096, dtype=torch.float32, device="cuda")
    with pytest.raises(d.DMuonError):
        d.diag_mix("prep", a, b, a)  # c is a
