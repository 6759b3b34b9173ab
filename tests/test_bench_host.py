"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the flop
accounting behind ``value``, ``executed_tflops`` and the roofline, and the
check that ties a committed counter summary to the kernel source it was taken
on."""

import hashlib
import os

import pytest

import bench
from matrix_optimizer_02_amd.workloads import get_workload


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_owner_share_shapes_and_flop_totals():
    """The Llama-3.1-8B owner share is 12 matrices of 4096 x 14336 (either
    orientation), 8 of 4096 x 4096 and 8 of 1024 x 4096 (short side first).
    Its short-side work over 5 iterations, counted by hand per shape class:
    Gram triangle m(m+1)n, A A^T triangle m(m+1)m, dense B X 2 m^2 n."""
    w = get_workload("llama3.1-8b_owner_1of8")
    shapes = sorted((min(s.rows, s.cols), max(s.rows, s.cols)) for s in w.matrices)
    assert shapes == sorted([(4096, 14336)] * 12 + [(4096, 4096)] * 8 + [(1024, 4096)] * 8)
    by_hand = 0
    for m, n, k in ((4096, 14336, 12), (4096, 4096, 8), (1024, 4096, 8)):
        by_hand += k * 5 * (m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n)
    total = sum(bench.NS_STEPS * bench.algorithmic_flops(m, n) for m, n in shapes)
    assert total == by_hand
    assert abs(total / 1e12 - 58.98) < 0.01
    dense = sum(bench.NS_STEPS * bench.dense_flops(m, n) for m, n in shapes)
    assert abs(dense / 1e12 - 83.24) < 0.01


@pytest.mark.parametrize("m,n", [(4096, 14336), (1024, 4096), (128, 512), (96, 96)])
def test_segment_of_one_counts_the_short_side(m, n):
    ex = bench.executed_flops(m, n, 1)
    assert ex["prod"] == 0
    assert sum(ex.values()) == bench.NS_STEPS * bench.algorithmic_flops(m, n)


def test_gram_space_counts_by_hand():
    """Restart after 3: segments of 3 and 2 iterations.  Per segment one Gram
    triangle, one square per iteration, three m x m triangles per iteration
    but the last (P' = Q P, T = A Q, A' = Q T) and one B X."""
    m, n = 1024, 4096
    tri_n, tri_m = m * (m + 1) * n, m * (m + 1) * m
    ex = bench.executed_flops(m, n, 3)
    assert ex == {"gram": 2 * tri_n, "square": 5 * tri_m, "prod": (3 * 2 + 3 * 1) * tri_m,
                  "bx": 2 * 2 * m * m * n}
    # a segment as long as the loop: one Gram, one B X
    ex5 = bench.executed_flops(m, n, 5)
    assert ex5["gram"] == tri_n and ex5["bx"] == 2 * m * m * n and ex5["prod"] == 12 * tri_m


def test_traffic_summary_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "matrix_optimizer_02_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "k_gemm_bf16.hip"
    src.write_text("// kernel v1\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "k_traffic.txt").write_text(
        f"kernel_source_sha256: {sha}\nhbm_bytes_per_launch: 6.25e9\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("k") == 6.25e9
    src.write_text("// kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.read_traffic("k") is None
    assert bench.read_traffic("missing") is None


def test_committed_traffic_summary_parses():
    path = os.path.join(bench.ROOT, "profiles", "bx_gemm_bf16_llama8b_traffic.txt")
    text = open(path).read()
    assert "kernel_source_sha256:" in text and "hbm_bytes_per_launch:" in text


def test_resident_counts_whole_products():
    m, n = 100, 400
    ex = bench.executed_flops(m, n, 1, resident=True)
    assert ex == {"gram": 5 * 2 * m * m * n, "square": 5 * 2 * m ** 3, "prod": 0, "bx": 5 * 2 * m * m * n}


def test_bx_flops_by_iteration():
    # a matrix's closing product runs where its segments end; resident ones none
    from matrix_optimizer_02_amd.workloads import custom_workload

    w = custom_workload("t", [(256, 1024), (512, 512), (1024, 256), (128, 256)])
    by = bench.bx_flops_by_iteration(w, [3, 1, 2, 1], [False, False, False, True])
    a, b, c = bench.bx_flops(256, 1024), bench.bx_flops(512, 512), bench.bx_flops(256, 1024)
    assert by == [b, b + c, a + b, b + c, a + b + c]
    # the per-phase totals agree with executed_flops
    tot = sum(bench.executed_flops(min(s.rows, s.cols), max(s.rows, s.cols), L)["bx"]
              for s, L in zip(w.matrices[:3], [3, 1, 2]))
    assert sum(by) == tot


def test_dominant_kernel_choice():
    rows = [[1.0, 2.0, 3.0, 4.0, 5.0], [1.0, 2.0, 3.0, 4.0, 5.0]]
    # a short-side bucket: B X launches in iterations 0 .. 4
    k, ms, fl, it = bench.dominant_kernel([10, 10, 10, 10, 10], False, 0, rows, 9.0, False)
    assert "bf16" in k and ms == 3.0 and fl == 10.0 and it == [0, 1, 2, 3, 4]
    # Gram space only, every 3 iterations: segments close in iterations 2 and 4
    k, ms, fl, it = bench.dominant_kernel([0, 0, 20, 0, 20], False, 0, rows, 9.0, False)
    assert ms == 4.0 and fl == 20.0 and it == [2, 4]
    # the last launch writes the updates: an instance of its own, timed apart
    k, ms, fl, it = bench.dominant_kernel([10, 10, 30, 10, 40], True, 0, rows, 9.0, False)
    assert ms == 2.5 and fl == 15.0 and it == [0, 1, 2, 3] and "plain" in k
    # ... unless it is the only one
    k, ms, fl, it = bench.dominant_kernel([0, 0, 0, 0, 20], True, 0, rows, 9.0, False)
    assert ms == 5.0 and fl == 20.0 and it == [4]
    # fp32 only: the fp32 matrix-core kernel
    k, ms, fl, it = bench.dominant_kernel([10, 10, 10, 10, 10], False, 0, rows, 9.0, True)
    assert "f32" in k and ms == 3.0
    # every bucket resident: the resident launch, timed inside iteration 0's Gram phase
    k, ms, fl, it = bench.dominant_kernel([0, 0, 0, 0, 0], False, 7.0, rows, 9.0, False)
    assert "resident" in k and ms == 9.0 and fl == 7.0 and it == []