"""Benchmark of the owner-side Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one muon_step_batched call over the whole matrix set: momentum,
normalisation, 5 quintic Newton-Schulz iterations on the short side and the
parameter update, with every input already resident in device memory.  The
default workload is the Llama-3.1-8B projection set's owner share (one of 8 LPT
owners: 28 matrices, bf16 gradients and parameters, fp32 momentum).

Printed: one JSON line.  ``value`` is the Newton-Schulz throughput of the
whole step in the flops its kernels execute: the short-side recurrence's
5 (m(m+1)n + m(m+1)m + 2 m^2 n) per matrix (the Gram and A A^T triangles plus
the dense B X product), or, for buckets that run the Gram-space form, that
form's 6 m^2 n + 14 m^3 over 5 iterations with a restart after 3
(9 m^2 n + 11 m^3 with restarts every 2), triangles halved -- divided by the
step time.  ``pct_bf16_peak`` is ``value`` over the 2.5 PFLOP/s bf16 dense
peak, the matrix-core utilisation of the step.  ``effective_tflops`` counts
the short-side recurrence's flops for every matrix whichever form runs (a
fixed amount of work per workload, above what the matrix cores execute when
the Gram space runs).
``roofline`` covers the dominant kernel, the B X product, timed live with HIP
events at its launch boundaries inside the timed steps.
``elementwise`` gives the bandwidth-bound passes of the same steps (prep:
momentum, cast and norm partials; apply: the update of the matrices that the
last B X launch does not update from its epilogue -- on the bf16 owner shares,
none) in GB/s of their required traffic against the 8 TB/s HBM peak;
``update_in_last_bx`` counts the updates written by that epilogue.  ``adamw`` times the AdamW companion
step on Llama-3.1-8B's non-Muon parameters (one GPU's 1/8 element share) the
same way.  ``graph`` replays the same step from a HIP graph (no host enqueueing
in the timed span; the number that matters for small, launch-bound
workloads).  ``step_ms_median`` and ``step_ms_min`` are the steps' device
times from their first to their last event.  ``torch_baseline`` times the same
step written with PyTorch matrix products (hipBLASLt) on the same inputs, for
context.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of
the same workload (one matrix per distinct shape and orientation) and
extrapolates it to the whole set by multiplicity, with single-thread oracle
times of the two small workloads.  ``small_workloads`` gives those two
workloads' graph-replayed step times on the GPU.  ``power`` samples the socket
power through amdsmi during the timed steps; ``clock`` is the shader clock read
by the library's sampler kernel over as many steps again, in a pass of its own.
``ceilings`` measures, in the same run, what the chip sustains outside this
library: a streaming copy (the practical HBM ceiling), each bandwidth-bound
pass's own byte mix (dtypes, streams, read/write ratio) on flat contiguous
arrays, and a matrix-core burn on pseudo-random bf16 operands with no memory
traffic (the bf16 rate the power limit allows); the roofline and the
elementwise passes are also given as fractions of these.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix (v_mfma_f32_*_f32)
HBM_PEAK_BPS = 8.0e12       # MI355X HBM3E
NS_STEPS = 5
LR, BETA, EPS = 0.02, 0.95, 1e-7


def algorithmic_flops(m: int, n: int) -> int:
    """One NS iteration: Gram triangle m(m+1)n, A A^T triangle m(m+1)m, B X 2m^2 n."""
    return m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n


def dense_flops(m: int, n: int) -> int:
    return 4 * m * m * n + 2 * m * m * m


def bx_flops(m: int, n: int) -> int:
    return 2 * m * m * n


def executed_flops(m: int, n: int, seg_len: int, steps: int = NS_STEPS, resident: bool = False) -> dict:
    """Flops one matrix's iterations perform, per phase kind, on the real
    shape with triangles halved as the kernels compute them.  The iterations
    run as segments of seg_len (1: the short side; the last segment shorter);
    a segment of L iterations takes one Gram product, L squares, 3 (L - 1)
    m x m triangles (P' = Q P, T = A Q, A' = Q T) and one B X product.  A
    resident bucket (every iteration in one workgroup) computes X X^T and A A
    whole."""
    tri_n, tri_m = m * (m + 1) * n, m * (m + 1) * m
    if resident:
        tri_n, tri_m = 2 * m * m * n, 2 * m * m * m
    segs = [seg_len] * (steps // seg_len) + ([steps % seg_len] if steps % seg_len else [])
    out = {"gram": 0, "square": 0, "prod": 0, "bx": 0}
    for L in segs:
        out["gram"] += tri_n
        out["square"] += L * tri_m
        out["prod"] += 3 * (L - 1) * tri_m
        out["bx"] += bx_flops(m, n)
    return out


def bx_flops_by_iteration(w, seg_len, resident, steps: int = NS_STEPS):
    """B X flops of each iteration's grouped launch: a matrix's closing product
    runs in the iterations that end one of its segments (every iteration on
    the short side; the last segment may be shorter)."""
    out = [0] * steps
    for s, L, res in zip(w.matrices, seg_len, resident):
        if res:
            continue
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        for k in range(steps):
            if k % L == L - 1 or k == steps - 1:
                out[k] += bx_flops(m, n)
    return out


def dominant_kernel(bx_by_iter, any_fused, res_flops, bx_ms_per_step, gram0_ms, f32_only, steps: int = NS_STEPS):
    """(kernel name, average launch ms, flops per launch, iterations timed) of
    the kernel the roofline covers.  With any bucket in the grouped launches it
    is the B X product: its launches are the iterations that close a segment of
    such a bucket, one grouped launch per tile class.  When the last of them
    also writes parameter updates (any_fused) it is an instance of its own,
    timed apart, and the roofline covers the plain ones (unless it is the only
    one).  With every bucket resident it is the resident kernel, one launch per
    step, timed inside iteration 0's Gram phase.  bx_ms_per_step holds each
    timed step's B X phase times."""
    bx_iters = [k for k in range(steps) if bx_by_iter[k] > 0]
    if bx_iters:
        plain = [k for k in bx_iters if not (any_fused and k == steps - 1)] or bx_iters
        bx_ms = [row[k] for row in bx_ms_per_step for k in plain]
        kernel = ("ns_gemm_f32_kernel<BX> (X' = s (a X + B X), fp32 MFMA)" if f32_only
                  else "ns_gemm_bf16_kernel<256, BX> (X' = s B' X, B' = aI + B)" + (
                      "; the plain launches (the last one, writing the updates, is timed apart)"
                      if any_fused and len(plain) < len(bx_iters) else ""))
        return kernel, sum(bx_ms) / len(bx_ms), sum(bx_by_iter[k] for k in plain) / len(plain), plain
    return ("ns_resident_kernel (every iteration of a small bf16 bucket in one launch, the matrix in LDS)",
            gram0_ms, res_flops, [])


def read_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (sha256 recorded in the summary)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    src = os.path.join(ROOT, "matrix_optimizer_02_amd", "csrc", "k_gemm_bf16.hip")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return float(m_b.group(1))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def multiplicity(w):
    """Count of each distinct (rows, cols) of a workload, in first-appearance order."""
    mult = {}
    for s in w.matrices:
        mult[(s.rows, s.cols)] = mult.get((s.rows, s.cols), 0) + 1
    return mult


def cpu_baseline(w, host_samples, gpu_ms_per_step):
    """Time the fp64 oracle (a dense Muon step per matrix, numpy on the host's
    BLAS threads) on one matrix per distinct (rows, cols) of the workload, and
    extrapolate to the whole set by multiplicity."""
    import oracle

    cores = _blas_threads()
    mult = multiplicity(w)
    alg = dense = 0
    per_shape = {}
    t_all = time.perf_counter()
    for i, (g, mm, ww) in host_samples:
        spec = w.matrices[i]
        t0 = time.perf_counter()
        oracle.muon_step(g, mm, ww, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS)
        per_shape[(spec.rows, spec.cols)] = time.perf_counter() - t0
        m, n = min(spec.rows, spec.cols), max(spec.rows, spec.cols)
        alg += NS_STEPS * algorithmic_flops(m, n)
        dense += NS_STEPS * dense_flops(m, n)
    dt = time.perf_counter() - t_all
    out = {"value": dense / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": "full fp64 oracle Muon step (numpy, dense products) on one matrix per distinct shape: "
                     + ", ".join(f"{r}x{c}" for r, c in per_shape) + f" ({dt:.1f} s)",
           "seconds": round(dt, 3),
           "value_counts": "flops the oracle executes: dense 4 m^2 n + 2 m^3 per iteration",
           "oracle_dense_flops_sample": dense,
           "effective_tflops": round(alg / dt / 1e12, 4)}
    if set(per_shape) == set(mult):
        whole = sum(per_shape[k] * mult[k] for k in mult)
        out["whole_set_seconds_extrapolated"] = round(whole, 2)
        out["extrapolation"] = ("sum over distinct (rows, cols) of the timed matrix's seconds times its "
                                "multiplicity: " + ", ".join(f"{r}x{c} x{mult[(r, c)]}" for r, c in mult))
        out["gpu_speedup_vs_oracle"] = round(whole / (gpu_ms_per_step / 1e3), 1)
    return out


def ceilings(d, dev, copy_bytes: int = 1 << 30, mfma_seconds: float = 0.5):
    """What the chip sustains outside the library, measured in this run: a
    streaming copy of copy_bytes (read + write bytes per second) and a
    matrix-core burn on pseudo-random bf16 operands for about mfma_seconds
    (after a warm-up of a fifth of that), with the clock read in a pass of its own."""
    import torch

    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        d.diag_copy(dst, src)
    e0.record()
    reps = 5
    for _ in range(reps):
        d.diag_copy(dst, src)
    e1.record()
    e1.synchronize()
    copy_bps = 2 * copy_bytes * reps / (e0.elapsed_time(e1) / 1e3)
    del src, dst
    # each bandwidth-bound pass's own byte mix, flat and contiguous, far beyond the 256 MB last-level cache
    mix = {}
    n_mix = 1 << 28
    for kind in ("prep", "apply", "adamw"):
        a = torch.zeros(n_mix, dtype=torch.bfloat16, device=dev)
        b = torch.zeros(n_mix, dtype=torch.float32 if kind == "prep" else torch.bfloat16, device=dev)
        c = (torch.zeros(n_mix, dtype=torch.bfloat16, device=dev) if kind == "prep" else
             torch.zeros(2 * n_mix, dtype=torch.float32, device=dev) if kind == "adamw" else None)
        for _ in range(2):
            nbytes = d.diag_mix(kind, a, b, c)
        e0.record()
        for _ in range(reps):
            d.diag_mix(kind, a, b, c)
        e1.record()
        e1.synchronize()
        bps = nbytes * reps / (e0.elapsed_time(e1) / 1e3)
        mix[kind] = {"elements": n_mix, "bytes_per_pass": nbytes, "tbps": round(bps / 1e12, 3),
                     "frac_hbm_peak": round(bps / HBM_PEAK_BPS, 4)}
        del a, b, c
    blocks = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    iters = 4096
    flops = d.diag_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    d.diag_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-4)
    n = max(10, int(mfma_seconds / per))
    for _ in range(max(2, n // 5)):
        d.diag_mfma(out, blocks, iters)
    power = PowerSampler()
    power.start()
    e0.record()
    for _ in range(n):
        d.diag_mfma(out, blocks, iters)
    e1.record()
    e1.synchronize()
    power.stop()
    seconds = e0.elapsed_time(e1) / 1e3
    mfma_tflops = flops * n / seconds / 1e12
    m = max(4, n // 2)

    def burn():
        for _ in range(m):
            d.diag_mfma(out, blocks, iters)

    clock = sample_clock(d, dev, burn, seconds * m / n)
    power_summary = power.summary()
    power.close()
    return {"copy": {"bytes_per_pass": 2 * copy_bytes, "tbps": round(copy_bps / 1e12, 3),
                     "frac_hbm_peak": round(copy_bps / HBM_PEAK_BPS, 4),
                     "kernel": "dmuon_diag_copy: streaming 16-byte loads and stores, four per lane in flight"},
            "mix": dict(mix, kernel="dmuon_diag_mix: each pass's dtypes, streams and read/write bytes on flat "
                                    "contiguous arrays, four 4-element groups per lane in flight"),
            "mfma_bf16": {"tflops": round(mfma_tflops, 1), "frac_bf16_peak": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
                          "launches": n, "seconds": round(seconds, 3),
                          "kernel": "dmuon_diag_mfma: v_mfma_f32_32x32x16_bf16 back to back on pseudo-random "
                                    "operands, no memory traffic",
                          "power": power_summary, "clock": clock}}


def small_workloads(d, dev, reps: int = 200, oracle_single_thread: bool = True):
    """The two small workloads (the fp32 256 x 512 matrix and the 96-matrix bf16
    batch): graph-replayed GPU step time and matrices/s, and the oracle's time
    for the same step on one host thread."""
    import torch

    from matrix_optimizer_02_amd.workloads import get_workload, make_inputs

    out = {}
    for name in ("f32_256x512", "bf16_small_batch_96"):
        w = get_workload(name)
        G, M, W = make_inputs(w, dev, seed=0)
        host = ([(g.double().cpu().numpy(), m.double().cpu().numpy(), x.double().cpu().numpy())
                 for g, m, x in zip(G, M, W)] if oracle_single_thread else None)
        plan = d.plan_for(G, [x.dtype for x in W])
        ws = d.workspace_for(plan, dev)
        for _ in range(3):
            d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS, workspace=ws)
        torch.cuda.synchronize()
        gr = graph_bench(d, plan, G, M, W, ws, reps, w.count)
        rec = {"matrices": w.count, "graph_us_per_step": round(gr["ms_per_step"] * 1e3, 2),
               "matrices_per_s": gr["matrices_per_s"]}
        if host is not None:
            import oracle
            from threadpoolctl import threadpool_limits

            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                for g, m, x in host:
                    oracle.muon_step(g, m, x, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS)
                dt = time.perf_counter() - t0
            rec["oracle_single_thread_s"] = round(dt, 4)
            rec["gpu_speedup_vs_oracle_single_thread"] = round(dt / (gr["ms_per_step"] / 1e3), 1)
        out[name] = rec
        del G, M, W, ws
    return out


class PowerSampler:
    """Samples the socket power through amdsmi (the GPU metrics table the
    driver refreshes) on a host thread, every ``period`` seconds between
    start() and stop().  Records nothing but an error string where amdsmi is
    unavailable."""

    def __init__(self, period: float = 0.005):
        self.period = period
        self.samples = []
        self.error = None
        self._thread = None
        self._stop = None
        self._h = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self.perf_level = str(amdsmi.amdsmi_get_gpu_perf_level(self._h))
        except Exception as e:  # pragma: no cover - depends on the box
            self.error = f"{type(e).__name__}: {e}"

    @staticmethod
    def _num(v):
        return isinstance(v, (int, float)) and 0 < v < 10000

    def _loop(self):
        while not self._stop.is_set():
            try:
                m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                self.samples.append(m.get("current_socket_power"))
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading

        if self._h is None:
            return
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        pw = [v for v in self.samples if self._num(v)]
        out = {"source": f"amdsmi current_socket_power, sampled every {self.period * 1e3:.0f} ms",
               "perf_level": getattr(self, "perf_level", None), "samples": len(pw)}
        if pw:
            out.update({"mean_w": round(sum(pw) / len(pw), 1), "min_w": min(pw), "max_w": max(pw)})
        if self.error:
            out["error"] = self.error
        return out

    def close(self):
        if self._h is not None:
            try:
                self._amdsmi.amdsmi_shut_down()
            except Exception:  # pragma: no cover
                pass
            self._h = None


def sample_clock(d, dev, enqueue, expected_s: float):
    """The shader clock while ``enqueue()``'s work runs: the library's clock
    sampler (one wave reading the shader-clock counter against the 100 MHz wall
    clock) on a side stream of default priority, started just before the work
    and sized to end within it (90% of expected_s).  The wave takes a slot on
    one CU, which can hold back one workgroup of a full-chip launch, so this is
    a pass of its own beside the timed one; its own duration is returned too."""
    import torch

    span = max(0.9 * expected_s, 2e-3)
    samples = min(4096, max(2, int(span / 1e-3) + 1))
    interval = max(1, int(span * 1e8 / (samples - 1)))
    buf = torch.zeros(2 * samples, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    d.diag_clock(buf, samples, interval, stream=side)
    t0 = time.perf_counter()
    enqueue()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    v = buf.view(samples, 2).cpu().tolist()
    rates = [(c1 - c0) / (w1 - w0) * 100.0 for (c0, w0), (c1, w1) in zip(v, v[1:]) if w1 > w0]
    mean = (v[-1][0] - v[0][0]) / max(v[-1][1] - v[0][1], 1) * 100.0
    return {"source": "dmuon_diag_clock: shader-clock counter against the 100 MHz wall clock, one wave on a side "
                      "stream (the clock of the XCD it ran on)",
            "mean_mhz": round(mean, 1), "min_mhz": round(min(rates), 1) if rates else None,
            "max_mhz": round(max(rates), 1) if rates else None, "samples": samples,
            "interval_ms": round(interval / 1e5, 3), "pass_seconds": round(wall, 4),
            "bf16_peak_at_mean_mhz_tflops": round(BF16_PEAK_TFLOPS * mean / 2400.0, 1)}


def graph_bench(d, plan, G, M, W, ws, reps: int, count: int):
    """The same step captured once in a HIP graph and replayed: no host
    enqueueing in the timed span, which is what small, launch-bound workloads
    need.  Timed with HIP events around the replays on the current stream."""
    import torch

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"replays": reps, "ms_per_step": round(ms, 4), "matrices_per_s": round(count / (ms / 1e3), 2)}


def torch_baseline(G, M, W, steps: int = 3, warmup: int = 1):
    """The same step written with PyTorch tensor ops on the same GPU, the way a
    plain Muon implementation runs it: matrix by matrix, momentum and
    normalisation as tensor expressions and every Newton-Schulz iteration as
    three torch.mm products (hipBLASLt) on bf16 operands (fp32 on the fp32
    path), the full X X^T and A A included.  Timed with events on the current
    stream.  Context only: no part of the library runs here."""
    import torch

    a, b, c = 3.4445, -4.7750, 2.0315

    def step():
        for g, mo, p in zip(G, M, W):
            r, cols = p.shape
            mo.mul_(BETA).add_(g.float())
            u = g.float() + BETA * mo
            x = u.t() if r > cols else u
            x = (x / (x.norm() + EPS)).to(g.dtype).contiguous()
            for _ in range(NS_STEPS):
                A = torch.mm(x, x.t())
                B = b * A + c * torch.mm(A, A)
                x = a * x + torch.mm(B, x)
            o = x.t() if r > cols else x
            p.add_(o.to(p.dtype), alpha=-LR * max(1.0, r / cols) ** 0.5)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    e1.synchronize()
    return {"kind": "torch.mm per matrix (hipBLASLt), same inputs and GPU", "steps": steps,
            "ms_per_step": round(e0.elapsed_time(e1) / steps, 3)}


def adamw_bench(d, dev, steps: int = 10, warmup: int = 2):
    """The AdamW companion step on Llama-3.1-8B's non-Muon share, timed with
    HIP events on the current stream; bytes are the step's required traffic
    (bf16 p and g, fp32 m and v: 22 bytes per element)."""
    import torch

    from matrix_optimizer_02_amd.workloads import ADAMW_LLAMA8B_SHARE, adamw_inputs

    P, G, M, V = adamw_inputs(dev)
    n = sum(p.numel() for p in P)
    for t in range(warmup):
        d.adamw_step_batched(P, G, M, V, step=10 + t)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        d.adamw_step_batched(P, G, M, V, step=10 + warmup + t)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = n * (2 + 2 + 4 + 4 + 2 + 4 + 4)
    return {"workload": ADAMW_LLAMA8B_SHARE, "tensors": len(P), "elements": n, "ms": round(ms, 4),
            "bytes": nbytes, "gbps": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms / 1e3) / HBM_PEAK_BPS, 4)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3.1-8b_owner_1of8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-adamw", action="store_true", help="skip the AdamW companion measurement")
    ap.add_argument("--no-torch-baseline", action="store_true",
                    help="skip timing the same step written with PyTorch matrix products")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-small-workloads", action="store_true",
                    help="skip the two small workloads' graph-replayed step times")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the copy and matrix-core ceilings")
    ap.add_argument("--tuning-cache", default=None, metavar="PATH",
                    help="run the plan with per-shape tuning entries: loaded from PATH for this device, "
                         "or measured with muon_autotune on the benchmark inputs and saved there")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times): the reference "
                         "dispatch for scaling HBM traffic counters")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the owner-side step is one GPU's share of the work and the "
              "library runs no collectives; run it with --gpus 1", file=sys.stderr)
        return 2

    import torch

    from matrix_optimizer_02_amd import dmuon_ns as d
    from matrix_optimizer_02_amd.workloads import get_workload, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)
        return 0
    w = get_workload(args.workload)
    G, M, W = make_inputs(w, dev, seed=args.seed)
    paths = {s.grad_dtype for s in w.matrices}

    # bounded oracle sample: one matrix per distinct (rows, cols), smallest first, up to ~14 TFLOP
    # dense (about 25 s on 16 host threads)
    host_samples = []
    if not args.no_cpu_baseline:
        seen, budget = set(), 14e12
        order = sorted(range(w.count), key=lambda i: dense_flops(min(w.matrices[i].rows, w.matrices[i].cols),
                                                                 max(w.matrices[i].rows, w.matrices[i].cols)))
        for i in order:
            s = w.matrices[i]
            key = (s.rows, s.cols)
            cost = NS_STEPS * dense_flops(min(s.rows, s.cols), max(s.rows, s.cols))
            if key in seen or cost > budget:
                continue
            seen.add(key)
            budget -= cost
            host_samples.append((i, (G[i].double().cpu().numpy(), M[i].double().cpu().numpy(),
                                     W[i].double().cpu().numpy())))

    tuning, tuning_info = None, None
    if args.tuning_cache:
        tuning = d.load_tuning(args.tuning_cache)
        source = "loaded"
        if not tuning:
            t0 = time.perf_counter()
            tuning = d.autotune(G, [torch.float32] * len(G), reps=2)
            source = f"measured ({time.perf_counter() - t0:.1f} s)"
            d.save_tuning(tuning, args.tuning_cache)
        tuning_info = {"cache": args.tuning_cache, "device": d.device_key(), "source": source,
                       "entries": [e.to_dict() for e in tuning]}
    plan = d.plan_for(G, [x.dtype for x in W], tuning=tuning)
    ws = d.workspace_for(plan, dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS, workspace=ws)
    events = [d.PhaseEvents(NS_STEPS) for _ in range(args.steps)]
    power = PowerSampler()
    torch.cuda.synchronize()
    power.start()
    t0 = time.perf_counter()
    for k in range(args.steps):
        d.muon_step_batched_profiled(plan, G, M, W, events[k], lr=LR, beta=BETA, eps=EPS,
                                     workspace=ws, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    power.stop()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    names = events[0].names()
    per = [e.elapsed_ms() for e in events]
    step_gpu = sorted(sum(p) for p in per)  # first to last event of each step
    avg = {nm: sum(p[j] for p in per) / len(per) for j, nm in enumerate(names)}
    kind_of = lambda nm: re.sub(r"\d+$", "", nm)
    gemm_ms = [p[j] for p in per for j, nm in enumerate(names) if kind_of(nm) in ("gram", "square", "prod", "bx")]

    # the recurrence form the plan picked for each matrix's bucket (iterations per segment)
    seg_len = [plan.bucket(plan.query(i).bucket).gram_restart for i in range(w.count)]
    gram_space = [plan.bucket(plan.query(i).bucket).algo == d.ALGO_GRAM_SPACE for i in range(w.count)]
    resident = [plan.bucket(plan.query(i).bucket).resident for i in range(w.count)]
    # matrices whose update the kernel ending their iteration writes (the apply
    # pass skips them): the last B X launch, or the resident kernel
    fused = [plan.update_fused(i, NS_STEPS) for i in range(w.count)]
    fused_bx = [f and not r for f, r in zip(fused, resident)]
    fused_res = [f and r for f, r in zip(fused, resident)]
    alg = dense = 0
    execd = {"gram": 0, "square": 0, "prod": 0, "bx": 0}  # grouped launches
    res_flops = 0  # the resident kernel's (every iteration of a small bucket in one launch)
    for s, L, res in zip(w.matrices, seg_len, resident):
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        alg += NS_STEPS * algorithmic_flops(m, n)
        dense += NS_STEPS * dense_flops(m, n)
        for k, v in executed_flops(m, n, L, resident=res).items():
            if res:
                res_flops += v
            else:
                execd[k] += v
    executed = sum(execd.values()) + res_flops
    step_s = ms_per_step / 1e3
    value = executed / step_s / 1e12
    f32_only = paths == {"f32"}
    peak = FP32_PEAK_TFLOPS if f32_only else BF16_PEAK_TFLOPS
    phase_tot = {k: sum(p[j] for p in per for j, nm in enumerate(names) if kind_of(nm) == k) / len(per)
                 for k in execd}
    bx_by_iter = bx_flops_by_iteration(w, seg_len, resident)
    assert sum(bx_by_iter) == execd["bx"]
    bx_rows = [[p[names.index(f"bx{k}")] for k in range(NS_STEPS)] for p in per]
    kernel, launch_ms, flops_per_launch, bx_plain = dominant_kernel(
        bx_by_iter, any(fused_bx), res_flops, bx_rows, avg["gram0"], f32_only)
    achieved = flops_per_launch / (launch_ms / 1e3) / 1e12
    traffic = (read_traffic("bx_gemm_bf16_llama8b")
               if args.workload == "llama3.1-8b_owner_1of8" and not args.tuning_cache else None)

    out = {
        "metric": "NS TFLOP/s and % bf16 MFMA peak, Muon step ms for Llama-3-8B owner share",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(step_gpu[len(step_gpu) // 2], 4),
        "step_ms_min": round(step_gpu[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if paths == {"bf16"} else ("f32" if paths == {"f32"} else "bf16+f32"),
        "data": "synthetic (seeded normal gradients, momenta and parameters)",
        "config": {"workload": w.name, "matrices": w.count, "elements": w.elements(),
                   "ns_steps": NS_STEPS, "lr": LR, "beta": BETA, "nesterov": True},
        "value_counts": "flops the kernels execute (Gram-space buckets: that form's products; triangles halved)",
        "executed_flops_per_step": executed,
        "effective_tflops": round(alg / step_s / 1e12, 3),
        "effective_flops_per_step": alg,
        "pct_bf16_peak": round(100.0 * executed / step_s / 1e12 / BF16_PEAK_TFLOPS, 3),
        "ns_tflops_dense_equiv": round(dense / step_s / 1e12, 3),
        "recurrence": {"gram_space_matrices": sum(gram_space), "short_side_matrices": w.count - sum(gram_space),
                       "resident_matrices": sum(resident),
                       "gram_restart": {str(L): sum(1 for g, x in zip(gram_space, seg_len) if g and x == L)
                                        for L in sorted({x for g, x in zip(gram_space, seg_len) if g})}},
        "gemm_phases": {k: {"ms": round(phase_tot[k], 4), "executed_flops": execd[k],
                            "tflops": round(execd[k] / (phase_tot[k] / 1e3) / 1e12, 1) if phase_tot[k] > 0 else None}
                        for k in execd},
        "resident": ({"matrices": sum(resident), "executed_flops": res_flops,
                      "timed_in": "gram0 (its launch follows prep, before iteration 0's grouped Gram)"}
                     if res_flops else None),
        "matrices_per_s": round(w.count / step_s, 2),
        "phase_ms": {k: round(v, 4) for k, v in avg.items()},
        "gemm_ms_per_step": round(sum(gemm_ms) / len(per), 4),
        "roofline": {"bound": "mfma", "kernel": kernel,
                     "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "launch_ms": round(launch_ms, 4), "flops_per_launch": flops_per_launch,
                     "iterations": bx_plain},
    }
    # the bandwidth-bound passes of the same steps, against the HBM roofline
    elems = w.elements()
    gsz = 2 if paths == {"bf16"} else 4
    psz = 2 if all(s.param_dtype == "bf16" for s in w.matrices) else 4
    prep_bytes = elems * (gsz + 4 + 4 + gsz)   # read G, M; write M', U (as X)
    # the apply pass: read O (X), W; write W' -- for the matrices no other kernel updates
    psize = lambda s: 2 if s.param_dtype == "bf16" else 4
    apply_bytes = sum(s.rows * s.cols * (gsz + 2 * psize(s)) for s, f in zip(w.matrices, fused) if not f)
    fused_elems = sum(s.rows * s.cols for s, f in zip(w.matrices, fused_bx) if f)
    res_upd = [s for s, f in zip(w.matrices, fused_res) if f]

    def rate(nbytes, ms):
        if nbytes == 0 or ms <= 0:
            return {"gbps": None, "frac_hbm": None}
        return {"gbps": round(nbytes / (ms / 1e3) / 1e9, 1), "frac_hbm": round(nbytes / (ms / 1e3) / HBM_PEAK_BPS, 4)}

    out["elementwise"] = {
        "prep": {"bytes": prep_bytes, "ms": round(avg["prep"], 4), **rate(prep_bytes, avg["prep"])},
        "apply": {"bytes": apply_bytes, "ms": round(avg["apply"], 4), **rate(apply_bytes, avg["apply"]),
                  "matrices": w.count - sum(fused)},
        "update_in_last_bx": {"matrices": sum(fused_bx), "elements": fused_elems,
                              "bytes": fused_elems * 4,
                              "note": "read W, write W' (bf16) from the last B X launch's epilogue; "
                                      "the final X never goes to HBM, so the apply pass's 6 bytes "
                                      "per element become 4, inside that launch"},
        "update_in_resident": {"matrices": len(res_upd),
                               "elements": sum(s.rows * s.cols for s in res_upd),
                               "bytes": sum(s.rows * s.cols * 2 * psize(s) for s in res_upd),
                               "note": "read W, write W' from the resident kernel's final X in LDS, "
                                       "which also sums its matrices' norm partials: no finalize or "
                                       "apply launch for them"},
    }
    last = NS_STEPS - 1
    if any(fused_bx) and bx_by_iter[last] > 0 and last not in bx_plain:
        last_ms = sum(r[last] for r in bx_rows) / len(bx_rows)
        out["bx_update_launch"] = {
            "kernel": "ns_gemm_bf16_kernel<256, BX, fused update>: the last iteration's B X, whose epilogue "
                      "writes W' for the matrices it updates",
            "ms": round(last_ms, 4), "flops": bx_by_iter[last],
            "tflops": round(bx_by_iter[last] / (last_ms / 1e3) / 1e12, 1),
            "update_bytes": fused_elems * 4, "matrices": sum(fused_bx)}
    out["graph"] = graph_bench(d, plan, G, M, W, ws, max(args.steps, 50 if ms_per_step < 5 else 0), w.count)
    if tuning_info is not None:
        out["tuning"] = tuning_info
    if not args.no_torch_baseline:
        tb = torch_baseline(G, M, W)
        tb["library_speedup"] = round(tb["ms_per_step"] / ms_per_step, 3)
        out["torch_baseline"] = tb
    if not args.no_adamw:
        out["adamw"] = adamw_bench(d, dev)
    out["power"] = power.summary()
    power.close()

    def clocked_steps():
        for _ in range(args.steps):
            d.muon_step_batched(plan, G, M, W, lr=LR, beta=BETA, eps=EPS, ns_steps=NS_STEPS, workspace=ws)

    out["clock"] = sample_clock(d, dev, clocked_steps, ms_per_step * args.steps / 1e3)
    out["clock"]["pass"] = f"{args.steps} more steps after the timed ones, with the sampler beside them"
    if not args.no_ceilings:
        ce = ceilings(d, dev)
        out["ceilings"] = ce
        out["roofline"]["frac_of_sustained_mfma"] = (round(achieved / ce["mfma_bf16"]["tflops"], 4)
                                                     if not f32_only else None)
        for k in ("prep", "apply"):
            gb = out["elementwise"][k]["gbps"]
            out["elementwise"][k]["frac_of_copy"] = round(gb / (ce["copy"]["tbps"] * 1e3), 4) if gb else None
            out["elementwise"][k]["frac_of_mix"] = round(gb / (ce["mix"][k]["tbps"] * 1e3), 4) if gb else None
        if "adamw" in out:
            out["adamw"]["frac_of_copy"] = round(out["adamw"]["gbps"] / (ce["copy"]["tbps"] * 1e3), 4)
            out["adamw"]["frac_of_mix"] = round(out["adamw"]["gbps"] / (ce["mix"]["adamw"]["tbps"] * 1e3), 4)
    if not args.no_small_workloads and args.workload not in ("f32_256x512", "bf16_small_batch_96"):
        out["small_workloads"] = small_workloads(d, dev, oracle_single_thread=not args.no_cpu_baseline)
    if host_samples:
        out["cpu_baseline"] = cpu_baseline(w, host_samples, ms_per_step)
    for e in events:
        e.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
