"""Python binding of libdmuon_ns (ctypes): the C ABI's entry points under the
same names, plus argument marshalling.

Every step of the Muon path runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and the current torch stream into a
hipStream_t.  PyTorch provides device memory and streams, nothing else.  If the
library is not built, importing this module raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import dataclasses
import json
import os
from typing import Dict, List, Optional, Sequence

import torch  # loads the HIP runtime the library binds to

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdmuon_ns.so")

DMUON_OK = 0
DMUON_ERR_INVALID_ARG = -1
DMUON_ERR_UNSUPPORTED = -2
DMUON_ERR_WORKSPACE = -3
DMUON_ERR_HIP = -4
DMUON_ERR_ALLOC = -5

DMUON_F32 = 0
DMUON_BF16 = 1

_DTYPE_CODE = {torch.float32: DMUON_F32, torch.bfloat16: DMUON_BF16,
               "f32": DMUON_F32, "bf16": DMUON_BF16}
_CODE_DTYPE = {DMUON_F32: torch.float32, DMUON_BF16: torch.bfloat16}


class DMuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class MatrixDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("grad_dtype", ctypes.c_int32), ("param_dtype", ctypes.c_int32)]


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("eps", ctypes.c_float),
                ("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("nesterov", ctypes.c_int32)]


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


class TuneEntry(ctypes.Structure):
    """dmuon_tune_entry: how a plan runs a bucket of one (path, padded m, padded n)."""
    _fields_ = [("path", ctypes.c_int32), ("tile", ctypes.c_int32), ("padded_m", ctypes.c_int64),
                ("padded_n", ctypes.c_int64), ("algo", ctypes.c_int32), ("gram_restart", ctypes.c_int32),
                ("xcd_remap", ctypes.c_uint32), ("apply_pass", ctypes.c_int32),
                ("cost_ms_per_matrix", ctypes.c_double)]

    _KEYS = ("path", "tile", "padded_m", "padded_n", "algo", "gram_restart", "xcd_remap", "apply_pass",
             "cost_ms_per_matrix")
    _OPTIONAL = {"apply_pass": 0}  # keys a cache file may lack, with their default

    def to_dict(self) -> dict:
        return {k: getattr(self, k) for k in self._KEYS}

    @classmethod
    def from_dict(cls, d: dict) -> "TuneEntry":
        return cls(**{k: d[k] if k in d else cls._OPTIONAL[k] for k in cls._KEYS})

    def __repr__(self):
        return f"TuneEntry({self.to_dict()})"


XCD_REMAP_DEFAULT = 0xFFFFFFFF


class PlanOpts(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("gram_restart", ctypes.c_int32),
                ("tuned", ctypes.POINTER(TuneEntry)), ("tuned_count", ctypes.c_int32)]


# dmuon_algo
ALGO_AUTO, ALGO_SHORT_SIDE, ALGO_GRAM_SPACE = 0, 1, 2
_ALGO_CODE = {"auto": ALGO_AUTO, "short_side": ALGO_SHORT_SIDE, "gram_space": ALGO_GRAM_SPACE}


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python -m matrix_optimizer_02_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    c_int32_p = ctypes.POINTER(ctypes.c_int32)
    c_int64_p = ctypes.POINTER(ctypes.c_int64)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "muon_plan": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.c_int32, vpp]),
        "muon_plan_ex": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.c_int32, ctypes.POINTER(PlanOpts), vpp]),
        "muon_plan_bucket_algo": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, c_int32_p, c_int32_p]),
        "muon_plan_bucket_resident": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, c_int32_p]),
        "muon_plan_update_fused": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, c_int32_p]),
        "muon_plan_bucket_config": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(TuneEntry)]),
        "muon_autotune_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.c_int32,
                                                         ctypes.POINTER(PlanOpts), ctypes.POINTER(ctypes.c_size_t)]),
        "muon_autotune": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.c_int32, ctypes.POINTER(PlanOpts),
                                         vpp, vpp, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.POINTER(TuneEntry), ctypes.c_int32, c_int32_p]),
        "muon_plan_workspace_bytes": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
        "muon_plan_info": (ctypes.c_int, [ctypes.c_void_p, c_int32_p, c_int32_p]),
        "muon_plan_query": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, c_int32_p, c_int32_p,
                                           c_int32_p, c_int64_p, c_int64_p, c_int64_p]),
        "muon_plan_bucket": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, c_int32_p, c_int64_p,
                                            c_int64_p, c_int32_p, c_int32_p]),
        "muon_plan_destroy": (None, [ctypes.c_void_p]),
        "muon_step_batched": (ctypes.c_int, [ctypes.c_void_p, vpp, vpp, vpp, ctypes.POINTER(HParams),
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "ns_orthogonalize_batched": (ctypes.c_int, [ctypes.c_void_p, vpp, vpp, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                                    ctypes.c_void_p]),
        "muon_step_batched_profiled": (ctypes.c_int, [ctypes.c_void_p, vpp, vpp, vpp, ctypes.POINTER(HParams),
                                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                      vpp, ctypes.c_int32]),
        "muon_step_batched_noalloc": (ctypes.c_int, [ctypes.c_void_p, vpp, vpp, vpp, ctypes.POINTER(HParams),
                                                     ctypes.c_void_p]),
        "muon_step_event_count": (ctypes.c_int32, [ctypes.c_int32]),
        "dmuon_events_create": (ctypes.c_int, [ctypes.c_int32, vpp]),
        "dmuon_events_elapsed_ms": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.POINTER(ctypes.c_float)]),
        "dmuon_events_destroy": (ctypes.c_int, [ctypes.c_int32, vpp]),
        "adamw_step_batched": (ctypes.c_int, [ctypes.c_int32, c_int64_p, c_int32_p, c_int32_p, vpp, vpp, vpp,
                                              vpp, ctypes.POINTER(AdamWHParams), ctypes.c_void_p]),
        "dmuon_diag_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "dmuon_diag_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
        "dmuon_diag_clock": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
        "dmuon_diag_mix": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]),
        "dmuon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dmuon_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def status_string(status: int) -> str:
    return _lib.dmuon_status_string(int(status)).decode()


def version() -> str:
    return _lib.dmuon_version().decode()


def _check(status: int, where: str):
    if status != DMUON_OK:
        raise DMuonError(status, where)


@dataclasses.dataclass(frozen=True)
class PlanEntry:
    bucket: int
    slot: int
    transposed: bool
    padded_m: int
    padded_n: int
    ns_cost: int


@dataclasses.dataclass(frozen=True)
class BucketEntry:
    path: int
    padded_m: int
    padded_n: int
    count: int
    tile: int
    algo: int          # ALGO_SHORT_SIDE | ALGO_GRAM_SPACE
    gram_restart: int  # iterations per Gram-space segment (1 on the short side)
    resident: bool     # every iteration in one workgroup per matrix, in LDS


class Plan:
    """Owner of a dmuon_plan (host memory only)."""

    def __init__(self, descs: Sequence[tuple], algo="auto", gram_restart: int = 0,
                 tuning: Optional[Sequence[TuneEntry]] = None):
        """descs: (rows, cols, grad_dtype, param_dtype); dtypes as torch dtypes,
        "bf16"/"f32" or the DMUON_* codes.  algo: "auto", "short_side" or
        "gram_space" (or the ALGO_* codes); gram_restart: Gram-space
        iterations between restarts (0: the library's default); tuning:
        per-shape entries (see autotune, load_tuning)."""
        self.descs = [(int(r), int(c), _code(g), _code(p)) for (r, c, g, p) in descs]
        arr = _desc_array(self.descs)
        handle = ctypes.c_void_p()
        self._destroy = _lib.muon_plan_destroy
        opts = _plan_opts(algo, gram_restart, tuning)
        _check(_lib.muon_plan_ex(arr, len(self.descs), ctypes.byref(opts), ctypes.byref(handle)), "muon_plan_ex")
        self._h = handle
        # what every call checks its tensors against (the descriptors are valid now), computed once
        self._sizes = [torch.Size((d[0], d[1])) for d in self.descs]
        self._dtypes = {"grad": [_CODE_DTYPE[d[2]] for d in self.descs],
                        "param": [_CODE_DTYPE[d[3]] for d in self.descs],
                        "momentum": [torch.float32] * len(self.descs)}

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def __len__(self):
        return len(self.descs)

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(_lib.muon_plan_workspace_bytes(self._h, ctypes.byref(n)), "muon_plan_workspace_bytes")
        return n.value

    def info(self):
        c, b = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.muon_plan_info(self._h, ctypes.byref(c), ctypes.byref(b)), "muon_plan_info")
        return c.value, b.value

    def query(self, idx: int) -> PlanEntry:
        b, s, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        pm, pn, cost = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(_lib.muon_plan_query(self._h, int(idx), ctypes.byref(b), ctypes.byref(s), ctypes.byref(t),
                                    ctypes.byref(pm), ctypes.byref(pn), ctypes.byref(cost)),
               "muon_plan_query")
        return PlanEntry(b.value, s.value, bool(t.value), pm.value, pn.value, cost.value)

    def bucket(self, b: int) -> BucketEntry:
        path, cnt, tile = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        pm, pn = ctypes.c_int64(), ctypes.c_int64()
        _check(_lib.muon_plan_bucket(self._h, int(b), ctypes.byref(path), ctypes.byref(pm), ctypes.byref(pn),
                                     ctypes.byref(cnt), ctypes.byref(tile)), "muon_plan_bucket")
        algo, restart = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.muon_plan_bucket_algo(self._h, int(b), ctypes.byref(algo), ctypes.byref(restart)),
               "muon_plan_bucket_algo")
        res = ctypes.c_int32()
        _check(_lib.muon_plan_bucket_resident(self._h, int(b), ctypes.byref(res)), "muon_plan_bucket_resident")
        return BucketEntry(path.value, pm.value, pn.value, cnt.value, tile.value, algo.value, restart.value,
                           bool(res.value))

    def update_fused(self, idx: int, ns_steps: int = 5) -> bool:
        """Whether a step of ns_steps iterations writes matrix idx's update from
        the kernel that ends its iteration, the resident kernel or its last B X
        launch (else the separate apply pass writes it)."""
        res = ctypes.c_int32()
        _check(_lib.muon_plan_update_fused(self._h, int(idx), int(ns_steps), ctypes.byref(res)),
               "muon_plan_update_fused")
        return bool(res.value)

    def config(self, b: int) -> TuneEntry:
        """The configuration bucket b runs with, as a tuning entry."""
        e = TuneEntry()
        _check(_lib.muon_plan_bucket_config(self._h, int(b), ctypes.byref(e)), "muon_plan_bucket_config")
        return e

    def close(self):
        # no module globals here: this also runs from __del__ at interpreter exit
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
        self._h = None

    def __del__(self):
        self.close()


def _desc_array(descs):
    arr = (MatrixDesc * max(1, len(descs)))()
    for i, (r, c, g, p) in enumerate(descs):
        arr[i] = MatrixDesc(r, c, g, p)
    return arr


def _plan_opts(algo, gram_restart, tuning) -> PlanOpts:
    opts = PlanOpts(algo if isinstance(algo, int) else _ALGO_CODE[algo], int(gram_restart))
    if tuning:
        tab = (TuneEntry * len(tuning))(*tuning)
        opts.tuned = ctypes.cast(tab, ctypes.POINTER(TuneEntry))
        opts.tuned_count = len(tuning)
        opts._keep = tab  # alive for the call
    return opts


def _code(d) -> int:
    if isinstance(d, int):
        return d
    return _DTYPE_CODE[d]


def muon_plan(descs: Sequence[tuple], algo="auto", gram_restart: int = 0,
              tuning: Optional[Sequence[TuneEntry]] = None) -> Plan:
    return Plan(descs, algo, gram_restart, tuning)


def plan_for(tensors_or_shapes: Sequence, param_dtypes: Optional[Sequence] = None, algo="auto",
             gram_restart: int = 0, tuning: Optional[Sequence[TuneEntry]] = None) -> Plan:
    """Plan from gradient tensors (shape and dtype) and parameter dtypes."""
    descs = []
    for i, g in enumerate(tensors_or_shapes):
        pd = g.dtype if param_dtypes is None else param_dtypes[i]
        descs.append((g.shape[0], g.shape[1], g.dtype, pd))
    return Plan(descs, algo, gram_restart, tuning)


def workspace_for(plan: Plan, device=None) -> torch.Tensor:
    """A device byte buffer of the plan's workspace size (torch's allocator
    returns 256-byte aligned blocks)."""
    n = max(plan.workspace_bytes(), 1)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def _ptr_array(ts: Sequence[torch.Tensor]):
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def _on_current_device(t: torch.Tensor, what: str) -> None:
    # the library addresses memory of the device current on the calling thread
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what} is on {t.device}; the current device is cuda:{torch.cuda.current_device()}")


def _check_tensors(plan: Plan, ts: Sequence[torch.Tensor], which: str, kind: str):
    """Every tensor on the current device, contiguous, of its descriptor's
    shape and of the dtype `kind` ("grad", "param" or "momentum") gives it."""
    if len(ts) != len(plan.descs):
        raise ValueError(f"{which}: expected {len(plan.descs)} tensors, got {len(ts)}")
    dev = torch.cuda.current_device()
    for i, (t, size, want) in enumerate(zip(ts, plan._sizes, plan._dtypes[kind])):
        if t.get_device() != dev or t.dtype is not want or t.shape != size or not t.is_contiguous():
            _on_current_device(t, f"{which}[{i}]")
            if t.shape != size or not t.is_contiguous():
                raise ValueError(f"{which}[{i}]: expected contiguous {size[0]}x{size[1]}, got {tuple(t.shape)}")
            raise ValueError(f"{which}[{i}]: expected {want}, got {t.dtype}")


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def muon_step_batched(plan: Plan, grads: Sequence[torch.Tensor], momenta: Sequence[torch.Tensor],
                      params: Sequence[torch.Tensor], *, lr: float = 0.02, beta: float = 0.95,
                      weight_decay: float = 0.0, eps: float = 1e-7,
                      a: float = 3.4445, b: float = -4.7750, c: float = 2.0315, ns_steps: int = 5,
                      nesterov: bool = True, workspace: torch.Tensor = None, stream=None) -> None:
    """Enqueue one fused Muon step on ``stream`` (default: torch's current
    stream).  momenta and params are updated in place."""
    _check_tensors(plan, grads, "grads", "grad")
    _check_tensors(plan, momenta, "momenta", "momentum")
    _check_tensors(plan, params, "params", "param")
    if workspace is None:
        raise ValueError("workspace is required (see workspace_for)")
    _on_current_device(workspace, "workspace")
    hp = HParams(lr, beta, weight_decay, eps, a, b, c, int(ns_steps), 1 if nesterov else 0)
    g, m, p = _ptr_array(grads), _ptr_array(momenta), _ptr_array(params)
    st = _lib.muon_step_batched(plan.handle, ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p)),
                                ctypes.cast(m, ctypes.POINTER(ctypes.c_void_p)),
                                ctypes.cast(p, ctypes.POINTER(ctypes.c_void_p)), ctypes.byref(hp),
                                ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(st, "muon_step_batched")


# Bytes of the static device array muon_step_batched_noalloc uses as its
# workspace (DMUON_NOALLOC_SCRATCH_BYTES in the C header).
NOALLOC_SCRATCH_BYTES = 64 << 20


def muon_step_batched_noalloc(plan: Plan, grads: Sequence[torch.Tensor], momenta: Sequence[torch.Tensor],
                              params: Sequence[torch.Tensor], *, lr: float = 0.02, beta: float = 0.95,
                              weight_decay: float = 0.0, eps: float = 1e-7,
                              a: float = 3.4445, b: float = -4.7750, c: float = 2.0315, ns_steps: int = 5,
                              nesterov: bool = True, stream=None) -> None:
    """muon_step_batched without a workspace argument and without any
    allocation: the library's static per-GPU scratch array serves as the
    workspace, so the plan may need at most NOALLOC_SCRATCH_BYTES.  Calls on
    one GPU share that array and must not overlap in time."""
    _check_tensors(plan, grads, "grads", "grad")
    _check_tensors(plan, momenta, "momenta", "momentum")
    _check_tensors(plan, params, "params", "param")
    need = plan.workspace_bytes()
    if need > NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"the plan needs {need} bytes of workspace; muon_step_batched_noalloc holds "
                         f"{NOALLOC_SCRATCH_BYTES} (use muon_step_batched with a workspace)")
    hp = HParams(lr, beta, weight_decay, eps, a, b, c, int(ns_steps), 1 if nesterov else 0)
    g, m, p = _ptr_array(grads), _ptr_array(momenta), _ptr_array(params)
    vp = ctypes.POINTER(ctypes.c_void_p)
    st = _lib.muon_step_batched_noalloc(plan.handle, ctypes.cast(g, vp), ctypes.cast(m, vp), ctypes.cast(p, vp),
                                        ctypes.byref(hp), _stream_handle(stream))
    _check(st, "muon_step_batched_noalloc")


def ns_orthogonalize_batched(plan: Plan, inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor],
                             *, ns_steps: int = 5, a: float = 3.4445, b: float = -4.7750,
                             c: float = 2.0315, eps: float = 1e-7, workspace: torch.Tensor = None,
                             stream=None) -> None:
    """Enqueue outputs[i] = NS(inputs[i]) on ``stream``."""
    _check_tensors(plan, inputs, "inputs", "grad")
    _check_tensors(plan, outputs, "outputs", "param")
    if workspace is None:
        raise ValueError("workspace is required (see workspace_for)")
    _on_current_device(workspace, "workspace")
    i_arr, o_arr = _ptr_array(inputs), _ptr_array(outputs)
    st = _lib.ns_orthogonalize_batched(plan.handle, ctypes.cast(i_arr, ctypes.POINTER(ctypes.c_void_p)),
                                       ctypes.cast(o_arr, ctypes.POINTER(ctypes.c_void_p)),
                                       int(ns_steps), a, b, c, eps, ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream))
    _check(st, "ns_orthogonalize_batched")


def autotune(inputs: Sequence[torch.Tensor], out_dtypes: Optional[Sequence] = None, *, algo="auto",
             gram_restart: int = 0, ns_steps: int = 5, a: float = 3.4445, b: float = -4.7750,
             c: float = 2.0315, reps: int = 3, stream=None) -> List[TuneEntry]:
    """muon_autotune on these inputs (trial data, read only): one entry per
    bucket of the plan they form, the fastest measured configuration, with the
    Gram-space choices checked on the whole batch against the short side.
    Output buffers and the workspace are allocated here for the trials.
    Blocks."""
    out_dtypes = out_dtypes or [torch.float32] * len(inputs)
    descs = [(int(x.shape[0]), int(x.shape[1]), _code(x.dtype), _code(od)) for x, od in zip(inputs, out_dtypes)]
    for i, x in enumerate(inputs):
        _on_current_device(x, f"inputs[{i}]")
        if not x.is_contiguous() or x.dim() != 2:
            raise ValueError(f"inputs[{i}] must be a contiguous 2-D device tensor")
    arr = _desc_array(descs)
    opts = _plan_opts(algo, gram_restart, None)
    need = ctypes.c_size_t()
    _check(_lib.muon_autotune_workspace_bytes(arr, len(descs), ctypes.byref(opts), ctypes.byref(need)),
           "muon_autotune_workspace_bytes")
    dev = inputs[0].device if len(inputs) else None
    ws = torch.empty(max(1, need.value), dtype=torch.uint8, device=dev)
    outs = [torch.empty(x.shape, dtype=od, device=x.device) for x, od in zip(inputs, out_dtypes)]
    nb = Plan(descs, algo, gram_restart).info()[1]
    res = (TuneEntry * max(1, nb))()
    got = ctypes.c_int32()
    i_arr, o_arr = _ptr_array(inputs), _ptr_array(outs)
    vp = ctypes.POINTER(ctypes.c_void_p)
    st = _lib.muon_autotune(arr, len(descs), ctypes.byref(opts), ctypes.cast(i_arr, vp), ctypes.cast(o_arr, vp),
                            int(ns_steps), a, b, c, int(reps), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                            _stream_handle(stream), res, nb, ctypes.byref(got))
    _check(st, "muon_autotune")
    return [TuneEntry.from_dict(res[i].to_dict()) for i in range(got.value)]


def device_key(device=None) -> str:
    """Key a tuning cache by the device it was measured on."""
    p = torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device())
    return f"{getattr(p, 'gcnArchName', 'unknown')}/{p.name}/{p.multi_processor_count}cu"


def save_tuning(entries: Sequence[TuneEntry], path: str, key: Optional[str] = None) -> None:
    """Merge ``entries`` into the JSON cache at ``path`` under ``key`` (default:
    the current device); an entry replaces one with the same shape key."""
    key = key or device_key()
    data: Dict = {"format": 1, "devices": {}}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    cur = {(e["path"], e["padded_m"], e["padded_n"]): e for e in data["devices"].get(key, [])}
    for e in entries:
        cur[(e.path, e.padded_m, e.padded_n)] = e.to_dict()
    data["devices"][key] = sorted(cur.values(), key=lambda e: (e["path"], e["padded_m"], e["padded_n"]))
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1)
    os.replace(tmp, path)


def load_tuning(path: str, key: Optional[str] = None) -> List[TuneEntry]:
    """The entries cached at ``path`` for ``key`` (default: the current device);
    [] when the file or the key is absent."""
    if not os.path.exists(path):
        return []
    key = key or device_key()
    with open(path) as f:
        data = json.load(f)
    if data.get("format") != 1:
        raise ValueError(f"{path}: unknown tuning cache format")
    return [TuneEntry.from_dict(e) for e in data["devices"].get(key, [])]


def adamw_step_batched(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                       exp_avgs: Sequence[torch.Tensor], exp_avg_sqs: Sequence[torch.Tensor], *, step: int,
                       lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.01,
                       stream=None) -> None:
    """Enqueue one AdamW step over a list of tensors (updated in place):
    params bf16 or fp32, grads bf16 or fp32 of the same shape, fp32 moments.
    ``step`` counts from 1 and includes this step."""
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have the same length")
    for i in range(n):
        p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        for name, t in (("params", p), ("grads", g), ("exp_avgs", m), ("exp_avg_sqs", v)):
            _on_current_device(t, f"{name}[{i}]")
            if not t.is_contiguous():
                raise ValueError(f"{name}[{i}] must be a contiguous device tensor")
        if not (p.numel() == g.numel() == m.numel() == v.numel()):
            raise ValueError(f"tensor {i}: element counts differ")
        if p.dtype not in _DTYPE_CODE or g.dtype not in _DTYPE_CODE:
            raise ValueError(f"tensor {i}: params and grads must be float32 or bfloat16")
        if m.dtype != torch.float32 or v.dtype != torch.float32:
            raise ValueError(f"tensor {i}: moments must be float32")
    numels = (ctypes.c_int64 * max(1, n))(*[t.numel() for t in params])
    pdt = (ctypes.c_int32 * max(1, n))(*[_DTYPE_CODE[t.dtype] for t in params])
    gdt = (ctypes.c_int32 * max(1, n))(*[_DTYPE_CODE[t.dtype] for t in grads])
    hp = AdamWHParams(lr, betas[0], betas[1], eps, weight_decay, int(step))
    vp = ctypes.POINTER(ctypes.c_void_p)
    arrs = [ctypes.cast(_ptr_array(x), vp) for x in (params, grads, exp_avgs, exp_avg_sqs)]
    st = _lib.adamw_step_batched(n, numels, pdt, gdt, *arrs, ctypes.byref(hp), _stream_handle(stream))
    _check(st, "adamw_step_batched")


def diag_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Enqueue the streaming copy of src into dst (same byte size, a multiple of 16)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src must have the same byte size")
    _check(_lib.dmuon_diag_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n,
                                _stream_handle(stream)), "dmuon_diag_copy")


def diag_mfma(out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """Enqueue the matrix-core burn; returns the flops it performs.  out: fp32,
    at least blocks * 512 elements."""
    if out.dtype != torch.float32 or out.numel() < blocks * 512:
        raise ValueError("out must be fp32 with blocks * 512 elements")
    _check(_lib.dmuon_diag_mfma(ctypes.c_void_p(out.data_ptr()), int(blocks), int(iters), _stream_handle(stream)),
           "dmuon_diag_mfma")
    return 8 * blocks * iters * 8 * 32768


MIX_KINDS = {"prep": (0, 12), "apply": (1, 6), "adamw": (2, 22)}  # kind, bytes per element


def diag_mix(kind: str, a: torch.Tensor, b: torch.Tensor, c: Optional[torch.Tensor] = None, stream=None) -> int:
    """Enqueue the flat byte-mix kernel of one pass ('prep', 'apply' or
    'adamw'; a: bf16 n elements, b: fp32 for prep else bf16, n elements, c:
    bf16 n for prep, fp32 2 n for adamw, unused for apply).  Returns the bytes
    it moves."""
    k, per = MIX_KINDS[kind]
    n = a.numel()
    want_b = torch.float32 if kind == "prep" else torch.bfloat16
    if a.dtype != torch.bfloat16 or b.dtype != want_b or b.numel() != n:
        raise ValueError("a must be bf16 and b " + str(want_b) + " with as many elements")
    if kind == "prep" and (c is None or c.dtype != torch.bfloat16 or c.numel() != n):
        raise ValueError("prep: c must be bf16 with n elements")
    if kind == "adamw" and (c is None or c.dtype != torch.float32 or c.numel() != 2 * n):
        raise ValueError("adamw: c must be fp32 with 2 n elements")
    cp = ctypes.c_void_p(c.data_ptr()) if (c is not None and kind != "apply") else ctypes.c_void_p(0)
    _check(_lib.dmuon_diag_mix(k, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), cp, n,
                               _stream_handle(stream)), "dmuon_diag_mix")
    return per * n


def diag_clock(out: torch.Tensor, samples: int, interval_ticks: int, stream=None) -> None:
    """Enqueue the clock sampler: out int64 with 2 * samples elements, one
    (shader cycles, 100 MHz wall ticks) pair every interval_ticks."""
    if out.dtype != torch.int64 or not out.is_cuda or out.numel() < 2 * samples:
        raise ValueError("out must be a device int64 tensor with 2 * samples elements")
    _check(_lib.dmuon_diag_clock(ctypes.c_void_p(out.data_ptr()), int(samples), int(interval_ticks),
                                 _stream_handle(stream)), "dmuon_diag_clock")


class PhaseEvents:
    """HIP events for muon_step_batched_profiled: one set per step to time."""

    PHASES_PER_ITER = ("gram", "square", "prod", "bx")

    def __init__(self, ns_steps: int):
        self.ns_steps = int(ns_steps)
        self.n = _lib.muon_step_event_count(self.ns_steps)
        self.arr = (ctypes.c_void_p * self.n)()
        self._destroy = _lib.dmuon_events_destroy
        self._arr_p = ctypes.cast(self.arr, ctypes.POINTER(ctypes.c_void_p))
        _check(_lib.dmuon_events_create(self.n, self._arr_p), "dmuon_events_create")

    def names(self) -> List[str]:
        out = ["prep"]
        for it in range(self.ns_steps):
            out += [f"{p}{it}" for p in self.PHASES_PER_ITER]
        return out + ["apply"]

    def elapsed_ms(self) -> List[float]:
        """Per-phase milliseconds (waits for the last event)."""
        res = []
        for k in range(self.n - 1):
            ms = ctypes.c_float()
            _check(_lib.dmuon_events_elapsed_ms(self.arr[k], self.arr[k + 1], ctypes.byref(ms)),
                   "dmuon_events_elapsed_ms")
            res.append(ms.value)
        return res

    def close(self):
        if getattr(self, "arr", None) is not None:
            self._destroy(self.n, self._arr_p)
            self.arr = self._arr_p = None

    def __del__(self):
        self.close()


def muon_step_batched_profiled(plan: Plan, grads, momenta, params, events: PhaseEvents, *,
                               lr: float = 0.02, beta: float = 0.95, weight_decay: float = 0.0,
                               eps: float = 1e-7, a: float = 3.4445, b: float = -4.7750,
                               c: float = 2.0315, nesterov: bool = True,
                               workspace: torch.Tensor = None, stream=None) -> None:
    """muon_step_batched with a HIP event recorded at every phase boundary."""
    _check_tensors(plan, grads, "grads", "grad")
    _check_tensors(plan, momenta, "momenta", "momentum")
    _check_tensors(plan, params, "params", "param")
    if workspace is None:
        raise ValueError("workspace is required (see workspace_for)")
    _on_current_device(workspace, "workspace")
    hp = HParams(lr, beta, weight_decay, eps, a, b, c, events.ns_steps, 1 if nesterov else 0)
    g, m, p = _ptr_array(grads), _ptr_array(momenta), _ptr_array(params)
    vp = ctypes.POINTER(ctypes.c_void_p)
    st = _lib.muon_step_batched_profiled(plan.handle, ctypes.cast(g, vp), ctypes.cast(m, vp), ctypes.cast(p, vp),
                                         ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                                         workspace.numel() * workspace.element_size(), _stream_handle(stream),
                                         ctypes.cast(events.arr, vp), events.n)
    _check(st, "muon_step_batched_profiled")


class MuonBatch:
    """Convenience owner of a plan and its workspace for a fixed matrix set."""

    def __init__(self, grads: Sequence[torch.Tensor], params: Sequence[torch.Tensor], algo="auto",
                 gram_restart: int = 0, tuning: Optional[Sequence[TuneEntry]] = None):
        self.plan = plan_for(grads, [p.dtype for p in params], algo, gram_restart, tuning)
        self.workspace = workspace_for(self.plan, grads[0].device if len(grads) else None)

    def step(self, grads, momenta, params, **hp):
        muon_step_batched(self.plan, grads, momenta, params, workspace=self.workspace, **hp)

    def orthogonalize(self, inputs, outputs, **kw):
        ns_orthogonalize_batched(self.plan, inputs, outputs, workspace=self.workspace, **kw)


__all__ = ["Plan", "PlanEntry", "BucketEntry", "MuonBatch", "DMuonError", "PhaseEvents", "muon_plan",
           "plan_for", "workspace_for", "muon_step_batched", "muon_step_batched_profiled",
           "muon_step_batched_noalloc", "NOALLOC_SCRATCH_BYTES",
           "ns_orthogonalize_batched", "status_string",
           "version", "library_path", "DMUON_F32", "DMUON_BF16", "ALGO_AUTO", "ALGO_SHORT_SIDE",
           "ALGO_GRAM_SPACE", "PlanOpts", "TuneEntry", "XCD_REMAP_DEFAULT", "autotune", "device_key",
           "save_tuning", "load_tuning"]
