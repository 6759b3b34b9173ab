"""Seeded synthetic workloads: matrix shape sets and their input tensors.

This module holds the input recipe only -- shapes, dtypes, distributions and
seeds -- and none of the optimizer's arithmetic.  Both the library's tests and
the oracle's tests draw their inputs from here; neither side computes anything
here.

The pages measure on random initialisation and synthetic data (DMuon docs,
"基准测试" benchmark section), so every workload is synthetic:

* ``f32_256x512``          one fp32 256 x 512 gradient N(0, 1), zero momentum,
                            fp32 params N(0, 0.02^2)
* ``bf16_small_batch_96``  32 each of 128x128, 128x512, 512x128; bf16 grads
                            N(0, 1e-3^2), fp32 momentum N(0, 1e-3^2), bf16 params
                            N(0, 0.02^2)
* ``qwen2.5-1.5b_proj``    28 layers x {q 1536x1536, k 256x1536, v 256x1536,
                            o 1536x1536, gate 8960x1536, up 8960x1536,
                            down 1536x8960}
* ``llama3.1-8b_owner_1of8`` the Llama-3.1-8B projection set (32 layers x
                            {q 4096^2, k 1024x4096, v 1024x4096, o 4096^2,
                            gate 14336x4096, up 14336x4096, down 4096x14336})
                            LPT-partitioned by cost into 8 owners; owner 0's
                            share (28 matrices)
* ``qwen2.5-7b_proj``      28 layers x {q 3584^2, k 512x3584, v 512x3584,
                            o 3584^2, gate 18944x3584, up 18944x3584,
                            down 3584x18944}

Large sets use bf16 grads N(0, 1e-3^2), fp32 momentum N(0, 1e-3^2) and bf16
params N(0, 0.02^2).

Seeding: matrix ``idx`` of workload ``w`` and tensor kind (0 = gradient,
1 = momentum, 2 = parameter) draws from the key (seed, w.key, idx, kind).  Host
generation uses numpy's PCG64 seeded with ``SeedSequence(key)`` (fp32 normals,
then scaled, then rounded to bf16 where needed).  Device generation -- used for
the multi-GB sets -- uses torch's seeded generator on the device with the same
key folded into one 63-bit seed; tensors handed to the oracle are copied back
bit-exactly, so both sides always see the same values.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Sequence

import numpy as np

GRAD, MOMENTUM, PARAM = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int
    grad_dtype: str   # "bf16" | "f32"
    param_dtype: str  # "bf16" | "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    key: int                  # workload number folded into the seeds
    matrices: tuple           # tuple[MatrixSpec]
    g_std: float
    m_std: float              # 0.0: zero momentum buffers
    w_std: float

    @property
    def count(self) -> int:
        return len(self.matrices)

    def elements(self) -> int:
        return sum(s.rows * s.cols for s in self.matrices)


def dense_ns_cost(rows: int, cols: int) -> int:
    """Cost of one Newton-Schulz iteration on a rows x cols matrix, taken on its
    short side: 4 m^2 n + 2 m^3.  Used here only to split a model's matrix set
    between owners (the LPT share below), as the pages balance owners by
    computational cost (DMuon abstract)."""
    m, n = min(rows, cols), max(rows, cols)
    return 4 * m * m * n + 2 * m * m * m


def lpt_bins(costs: Sequence[int], nbins: int) -> List[List[int]]:
    """Longest-processing-time partition: stable sort by cost descending (input
    order breaks ties), each item to the least-loaded bin, lowest bin index on a
    tie.  The pages' owner assignment solves a MILP over profiled costs with a
    greedy fallback (explainer section 2.3); this greedy rule only picks which
    matrices form one owner's share."""
    order = sorted(range(len(costs)), key=lambda i: (-costs[i], i))
    loads = [0] * nbins
    bins: List[List[int]] = [[] for _ in range(nbins)]
    for i in order:
        b = min(range(nbins), key=lambda j: (loads[j], j))
        bins[b].append(i)
        loads[b] += costs[i]
    return [sorted(b) for b in bins]


def _layer_set(layers: int, shapes: Sequence[tuple], dtype: str = "bf16") -> List[MatrixSpec]:
    out = []
    for layer in range(layers):
        for nm, r, c in shapes:
            out.append(MatrixSpec(f"L{layer}.{nm}", r, c, dtype, dtype))
    return out


_QWEN15 = [("q", 1536, 1536), ("k", 256, 1536), ("v", 256, 1536), ("o", 1536, 1536),
           ("gate", 8960, 1536), ("up", 8960, 1536), ("down", 1536, 8960)]
_LLAMA8 = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
           ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
_QWEN7 = [("q", 3584, 3584), ("k", 512, 3584), ("v", 512, 3584), ("o", 3584, 3584),
          ("gate", 18944, 3584), ("up", 18944, 3584), ("down", 3584, 18944)]


def llama8b_full_set() -> List[MatrixSpec]:
    return _layer_set(32, _LLAMA8)


def llama8b_owner_share(owner: int = 0, owners: int = 8) -> List[MatrixSpec]:
    full = llama8b_full_set()
    bins = lpt_bins([dense_ns_cost(s.rows, s.cols) for s in full], owners)
    return [full[i] for i in bins[owner]]


def _build() -> dict:
    w = {}
    w["f32_256x512"] = Workload("f32_256x512", 1,
                                (MatrixSpec("g", 256, 512, "f32", "f32"),), 1.0, 0.0, 0.02)
    small = ([MatrixSpec(f"sq{i}", 128, 128, "bf16", "bf16") for i in range(32)]
             + [MatrixSpec(f"wide{i}", 128, 512, "bf16", "bf16") for i in range(32)]
             + [MatrixSpec(f"tall{i}", 512, 128, "bf16", "bf16") for i in range(32)])
    w["bf16_small_batch_96"] = Workload("bf16_small_batch_96", 2, tuple(small), 1e-3, 1e-3, 0.02)
    w["qwen2.5-1.5b_proj"] = Workload("qwen2.5-1.5b_proj", 3, tuple(_layer_set(28, _QWEN15)),
                                      1e-3, 1e-3, 0.02)
    w["llama3.1-8b_owner_1of8"] = Workload("llama3.1-8b_owner_1of8", 4,
                                           tuple(llama8b_owner_share(0, 8)), 1e-3, 1e-3, 0.02)
    w["qwen2.5-7b_proj"] = Workload("qwen2.5-7b_proj", 5, tuple(_layer_set(28, _QWEN7)),
                                    1e-3, 1e-3, 0.02)
    return w


WORKLOADS = _build()


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom_workload(name: str, shapes: Sequence[tuple], grad_dtype: str = "bf16",
                    param_dtype: str = "bf16", g_std: float = 1e-3, m_std: float = 1e-3,
                    w_std: float = 0.02, key: int = 100) -> Workload:
    """A test workload of arbitrary (rows, cols) shapes."""
    mats = tuple(MatrixSpec(f"m{i}", int(r), int(c), grad_dtype, param_dtype)
                 for i, (r, c) in enumerate(shapes))
    return Workload(name, key, mats, g_std, m_std, w_std)


def _seed_key(seed: int, wkey: int, idx: int, kind: int):
    return [int(seed), int(wkey), int(idx), int(kind)]


def _std_for(w: Workload, kind: int) -> float:
    return {GRAD: w.g_std, MOMENTUM: w.m_std, PARAM: w.w_std}[kind]


def _dtype_for(spec: MatrixSpec, kind: int) -> str:
    if kind == GRAD:
        return spec.grad_dtype
    if kind == MOMENTUM:
        return "f32"
    return spec.param_dtype


def host_normal(shape, std: float, key) -> np.ndarray:
    """fp32 N(0, std^2) from numpy PCG64 seeded by SeedSequence(key)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return (x * np.float32(std)).astype(np.float32)


def host_tensor(w: Workload, idx: int, kind: int, seed: int = 0):
    """CPU torch tensor of matrix ``idx`` and ``kind`` (fp32 or bf16)."""
    import torch

    spec = w.matrices[idx]
    std = _std_for(w, kind)
    if std == 0.0:
        x = np.zeros((spec.rows, spec.cols), dtype=np.float32)
    else:
        x = host_normal((spec.rows, spec.cols), std, _seed_key(seed, w.key, idx, kind))
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if _dtype_for(spec, kind) == "bf16" else t


def _fold_seed(key) -> int:
    h = hashlib.sha256(repr(tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def device_tensor(w: Workload, idx: int, kind: int, device, seed: int = 0):
    """Tensor of matrix ``idx`` and ``kind`` generated on ``device`` with torch's
    seeded generator (for multi-GB workloads)."""
    import torch

    spec = w.matrices[idx]
    dt = torch.bfloat16 if _dtype_for(spec, kind) == "bf16" else torch.float32
    std = _std_for(w, kind)
    if std == 0.0:
        return torch.zeros((spec.rows, spec.cols), dtype=dt, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(_fold_seed(_seed_key(seed, w.key, idx, kind)))
    x = torch.randn((spec.rows, spec.cols), generator=gen, dtype=torch.float32, device=device)
    x.mul_(std)
    return x.to(dt)


def make_inputs(w: Workload, device="cpu", seed: int = 0, on_device_gen: bool = None):
    """Lists (G, M, W) of tensors on ``device``.  Host generation (then a copy)
    unless ``on_device_gen`` (default: True for workloads above 64M elements)."""
    if on_device_gen is None:
        on_device_gen = w.elements() > (64 << 20) and str(device) != "cpu"
    Gs, Ms, Ws = [], [], []
    for i in range(w.count):
        for kind, lst in ((GRAD, Gs), (MOMENTUM, Ms), (PARAM, Ws)):
            if on_device_gen:
                lst.append(device_tensor(w, i, kind, device, seed))
            else:
                lst.append(host_tensor(w, i, kind, seed).to(device))
    return Gs, Ms, Ws


# ---- AdamW companion: the parameters that do not go through Muon -------------------
#
# Llama-3.1-8B's non-projection parameters -- token embedding and LM head
# (128256 x 4096 each, untied) and 65 RMSNorm weights of 4096 (two per layer
# plus the final one) -- split evenly between 8 GPUs as element shards, the
# way an element-wise optimizer's state is sharded.  One GPU's share: two
# shards of 65 667 072 and 65 shards of 512 elements, bf16 parameters and
# gradients, fp32 moments.  Parameters N(0, 0.02^2), gradients N(0, 1e-3^2),
# first moments N(0, 1e-4^2), second moments the square of N(0, 1e-3^2), at
# step 10.

ADAMW_LLAMA8B_SHARE = "llama3.1-8b_adamw_share_1of8"


def llama8b_adamw_share(owners: int = 8) -> List[tuple]:
    """(name, numel) of one GPU's shard of each non-Muon tensor."""
    vocab, hidden, layers = 128256, 4096, 32
    out = [("embed", vocab * hidden // owners), ("lm_head", vocab * hidden // owners)]
    out += [(f"norm{i}", hidden // owners) for i in range(2 * layers + 1)]
    return out


def adamw_inputs(device, seed: int = 0, owners: int = 8):
    """Lists (params, grads, exp_avgs, exp_avg_sqs) of the AdamW share, generated
    on ``device`` with torch's seeded generator, one key per (tensor, kind)."""
    import torch

    P, G, M, V = [], [], [], []
    for idx, (_, n) in enumerate(llama8b_adamw_share(owners)):
        def draw(kind, std):
            gen = torch.Generator(device=device)
            gen.manual_seed(_fold_seed((seed, 90, idx, kind)))
            return torch.randn(n, generator=gen, dtype=torch.float32, device=device).mul_(std)
        P.append(draw(PARAM, 0.02).to(torch.bfloat16))
        G.append(draw(GRAD, 1e-3).to(torch.bfloat16))
        M.append(draw(MOMENTUM, 1e-4))
        V.append(draw(3, 1e-3).square_())
    return P, G, M, V
