"""The C-ABI library on the host: it loads, exports every entry point the header
declares, its planner matches the planning rule's reference bit for bit, and
argument errors come back as status codes before any device work (no GPU is
touched by these tests)."""

import ctypes
import os

import pytest

from matrix_optimizer_02_amd import build as build_mod
from matrix_optimizer_02_amd import dmuon_ns as d
from matrix_optimizer_02_amd.workloads import WORKLOADS
from oracle import plan_reference

import torch

LIB = d._lib  # the typed entry points (argtypes set by the binding)
host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="fake device addresses: host-only validation test")


def test_exports_every_declared_symbol():
    raw = ctypes.CDLL(d.library_path())
    names = build_mod.exported_symbols()
    assert set(names) == {"muon_plan", "muon_plan_ex", "muon_plan_workspace_bytes", "muon_plan_info",
                          "muon_plan_query", "muon_plan_bucket", "muon_plan_bucket_algo", "muon_plan_bucket_config",
                          "muon_plan_bucket_resident", "muon_plan_update_fused",
                          "muon_autotune_workspace_bytes", "muon_autotune", "muon_plan_destroy",
                          "muon_step_batched", "muon_step_batched_noalloc",
                          "ns_orthogonalize_batched", "muon_step_batched_profiled", "muon_step_event_count",
                          "dmuon_events_create", "dmuon_events_elapsed_ms", "dmuon_events_destroy",
                          "adamw_step_batched", "dmuon_status_string", "dmuon_version",
                          "dmuon_diag_copy", "dmuon_diag_mfma", "dmuon_diag_clock",
                          "dmuon_diag_mix"}
    for n in names:
        assert hasattr(raw, n), n


def test_noalloc_scratch_size_matches_header():
    # the binding's copy of the static scratch size is the header's
    import re

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "include", "dmuon_ns.h")) as f:
        m = re.search(r"#define DMUON_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == d.NOALLOC_SCRATCH_BYTES


@host_only
def test_noalloc_host_errors_before_device_work():
    # size and null checks come before any HIP call (fake addresses never dereferenced)
    hp = d.HParams(0.02, 0.95, 0.0, 1e-7, 3.4445, -4.775, 2.0315, 5, 1)
    big = d.Plan([(4096, 4096, 1, 1)])  # 128 MiB of workspace
    assert big.workspace_bytes() > d.NOALLOC_SCRATCH_BYTES
    f = LIB.muon_step_batched_noalloc
    g = _arr([0x100000])
    assert f(big.handle, g, _arr([0x200000]), _arr([0x300000]), ctypes.byref(hp), None) == d.DMUON_ERR_WORKSPACE
    assert f(None, g, g, g, ctypes.byref(hp), None) == d.DMUON_ERR_INVALID_ARG
    assert f(big.handle, g, g, g, None, None) == d.DMUON_ERR_INVALID_ARG
    hp_bad = d.HParams(0.02, 0.95, 0.0, 1e-7, 3.4445, -4.775, 2.0315, -1, 1)
    assert f(big.handle, g, g, g, ctypes.byref(hp_bad), None) == d.DMUON_ERR_INVALID_ARG
    assert f(d.Plan([]).handle, None, None, None, ctypes.byref(hp), None) == d.DMUON_OK


def test_event_count():
    # prep, 4 phases per iteration (Gram, square, prod, B X), apply, and the start event
    assert LIB.muon_step_event_count(5) == 23 and LIB.muon_step_event_count(0) == 3
    assert LIB.muon_step_event_count(1) == 7
    assert LIB.muon_step_event_count(-1) == -1
    assert LIB.muon_step_event_count((2 ** 31 - 1 - 3) // 4) == 2 ** 31 - 1
    assert LIB.muon_step_event_count((2 ** 31 - 1 - 3) // 4 + 1) == -1


def test_status_strings_and_version():
    for code in (0, -1, -2, -3, -4, -5):
        assert d.status_string(code)
    assert d.status_string(7) == "unknown status"
    assert d.version().count(".") == 2


def _descs_of(w):
    code = {"bf16": 1, "f32": 0}
    return [(s.rows, s.cols, code[s.grad_dtype], code[s.param_dtype]) for s in w.matrices]


CASES = {
    "mixed_odd": [(300, 700, 1, 1), (700, 300, 1, 0), (100, 130, 1, 1), (256, 512, 0, 0), (65, 65, 0, 1),
                  (1, 513, 1, 1), (513, 1, 1, 1), (129, 129, 1, 1), (128, 129, 1, 1), (4096, 14336, 1, 1)],
    "ties": [(64, 64, 0, 0), (128, 128, 1, 1), (64, 64, 0, 0), (128, 128, 0, 0)],
}


ALGO = {"short_side": d.ALGO_SHORT_SIDE, "gram_space": d.ALGO_GRAM_SPACE}


@pytest.mark.parametrize("algo,restart", [("auto", 0), ("short_side", 0), ("gram_space", 0), ("gram_space", 2),
                                          ("auto", 5)])
@pytest.mark.parametrize("name", sorted(WORKLOADS) + sorted(CASES))
def test_plan_matches_reference(name, algo, restart):
    descs = CASES[name] if name in CASES else _descs_of(WORKLOADS[name])
    items, buckets = plan_reference(descs, algo, restart)
    p = d.Plan(descs, algo, restart)
    assert p.info() == (len(descs), len(buckets))
    for i, it in enumerate(items):
        e = p.query(i)
        assert (e.bucket, e.slot, e.transposed, e.padded_m, e.padded_n, e.ns_cost) == (
            it["bucket"], it["slot"], it["transposed"], it["m_pad"], it["n_pad"], it["cost"]), i
    for b, bk in enumerate(buckets):
        e = p.bucket(b)
        assert (e.path, e.padded_m, e.padded_n, e.count) == (
            0 if bk["path"] == "f32" else 1, bk["m_pad"], bk["n_pad"], len(bk["members"]))
        assert e.tile == (64 if bk["path"] == "f32" else (128 if bk["m_pad"] <= 128 else 256))
        assert (e.algo, e.gram_restart) == (ALGO[bk["algo"]], bk["gram_restart"]), b


def test_default_algo_by_hand():
    # bf16: Gram space exactly when the padded long side exceeds the padded short side,
    # the padded short side is at least 1024 and every member has n >= 3 m
    p = d.Plan([(4096, 14336, 1, 1), (4096, 4096, 1, 1), (1024, 4096, 0, 0), (1024, 4096, 1, 1),
                (200, 256, 1, 1), (128, 192, 1, 1), (100, 250, 1, 1), (384, 1000, 1, 1), (100, 700, 1, 1),
                (512, 120, 1, 1), (1100, 3000, 1, 1), (3400, 1100, 1, 1), (768, 3072, 1, 1)])
    got = {(p.bucket(b).padded_m, p.bucket(b).padded_n, p.bucket(b).path): p.bucket(b).algo
           for b in range(p.info()[1])}
    assert got == {(4096, 14336, 1): d.ALGO_GRAM_SPACE, (4096, 4096, 1): d.ALGO_SHORT_SIDE,
                   (1024, 4096, 0): d.ALGO_SHORT_SIDE, (1024, 4096, 1): d.ALGO_GRAM_SPACE,
                   (256, 256, 1): d.ALGO_SHORT_SIDE, (128, 256, 1): d.ALGO_SHORT_SIDE,
                   (512, 1024, 1): d.ALGO_SHORT_SIDE, (128, 768, 1): d.ALGO_SHORT_SIDE,
                   (128, 512, 1): d.ALGO_SHORT_SIDE, (1280, 3072, 1): d.ALGO_SHORT_SIDE,
                   (1280, 3584, 1): d.ALGO_GRAM_SPACE, (768, 3072, 1): d.ALGO_SHORT_SIDE}
    # one member with n < 3 m keeps its whole bucket on the short side
    p = d.Plan([(1100, 3400, 1, 1), (1150, 3400, 1, 1)])
    assert p.info()[1] == 1 and p.bucket(0).algo == d.ALGO_SHORT_SIDE


def test_tuned_gram_entry_respects_the_default_rule():
    # an entry's Gram space applies under the default option only where the default
    # rule would take it on the bucket's real members (entries are keyed by padded dims)
    e = d.TuneEntry(path=1, tile=0, padded_m=1280, padded_n=3584, algo=d.ALGO_GRAM_SPACE, gram_restart=2,
                    xcd_remap=d.XCD_REMAP_DEFAULT)
    assert d.Plan([(1100, 3400, 1, 1)], tuning=[e]).bucket(0).algo == d.ALGO_GRAM_SPACE
    assert d.Plan([(1150, 3400, 1, 1)], tuning=[e]).bucket(0).algo == d.ALGO_SHORT_SIDE
    assert d.Plan([(1150, 3400, 1, 1)], "gram_space", tuning=[e]).bucket(0).algo == d.ALGO_GRAM_SPACE


def test_default_restart_by_size():
    # Gram-space buckets restart every 2 iterations up to a padded short side of
    # 1024 and every 3 above; an explicit plan option or tuned entry overrides both
    descs = [(4096, 14336, 1, 1), (1024, 4096, 1, 1), (1100, 4000, 1, 1), (3072, 1024, 1, 1), (300, 700, 1, 1)]
    p = d.Plan(descs)
    got = {(p.bucket(b).padded_m, p.bucket(b).padded_n): p.bucket(b).gram_restart for b in range(p.info()[1])}
    assert got == {(4096, 14336): 3, (1024, 4096): 2, (1280, 4096): 3, (1024, 3072): 2, (512, 768): 1}
    q = d.Plan(descs, "gram_space", 4)
    assert {q.bucket(b).gram_restart for b in range(q.info()[1])} == {4}


def test_resident_buckets_by_hand():
    # bf16, padded short side 128, padded long side <= 512, on the short side
    descs = [(128, 128, 1, 1), (100, 250, 1, 1), (512, 120, 1, 0), (128, 513, 1, 1), (129, 300, 1, 1),
             (96, 160, 0, 0), (64, 64, 1, 1)]
    p = d.Plan(descs)
    got = {(p.bucket(b).padded_m, p.bucket(b).padded_n, p.bucket(b).path): p.bucket(b).resident
           for b in range(p.info()[1])}
    assert got == {(128, 128, 1): True, (128, 256, 1): True, (128, 512, 1): True, (128, 640, 1): False,
                   (256, 512, 1): False, (128, 192, 0): False}
    # forced onto every bf16 bucket, the Gram space leaves none resident
    g = d.Plan(descs, "gram_space")
    assert not any(g.bucket(b).resident for b in range(g.info()[1]))
    res = ctypes.c_int32()
    assert LIB.muon_plan_bucket_resident(None, 0, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_bucket_resident(p.handle, 99, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_bucket_resident(p.handle, 0, None) == d.DMUON_ERR_INVALID_ARG
    assert d.Plan([(128, 250, 1, 1), (128, 129, 1, 1)], "gram_space").bucket(0).algo == d.ALGO_GRAM_SPACE


def _entry(path, m_pad, n_pad, tile=0, algo=0, restart=0, remap=0xFFFFFFFF, cost=0.0, apply_pass=None):
    e = {"path": path, "padded_m": m_pad, "padded_n": n_pad, "tile": tile, "algo": algo,
         "gram_restart": restart, "xcd_remap": remap, "cost_ms_per_matrix": cost}
    if apply_pass is not None:  # absent: the field's default (entries of older caches lack it)
        e["apply_pass"] = apply_pass
    return e


TUNED_CASES = {
    # tile, form, restart and remap overrides on some buckets, dense-cost order kept
    "overrides": (CASES["mixed_odd"], [_entry(1, 512, 768, tile=128, remap=15), _entry(1, 256, 256, algo=2, restart=2),
                                       _entry(1, 4096, 14336, algo=1, remap=0, apply_pass=1),
                                       _entry(0, 256, 512, tile=64, apply_pass=0),
                                       _entry(1, 128, 640, restart=5), _entry(1, 999, 999, tile=128)]),
    # every bucket measured: ordered by count x cost, ties by first appearance
    "measured_order": ([(256, 512, 1, 1), (1024, 4096, 1, 1), (256, 512, 1, 1), (128, 128, 1, 1), (64, 64, 0, 0)],
                       [_entry(1, 256, 512, cost=2.0), _entry(1, 1024, 4096, cost=1.0), _entry(1, 128, 128, cost=4.0),
                        _entry(0, 64, 64, cost=4.0)]),
    # one bucket unmeasured: dense-cost order
    "partly_measured": ([(256, 512, 1, 1), (1024, 4096, 1, 1), (128, 128, 1, 1)],
                        [_entry(1, 256, 512, cost=9.0), _entry(1, 128, 128, cost=9.0)]),
}


def _tune_entries(es):
    return [d.TuneEntry.from_dict(e) for e in es]


@pytest.mark.parametrize("name", sorted(TUNED_CASES))
def test_tuned_plan_matches_reference(name):
    descs, es = TUNED_CASES[name]
    items, buckets = plan_reference(descs, tuned=es)
    p = d.Plan(descs, tuning=_tune_entries(es))
    assert p.info() == (len(descs), len(buckets))
    for i, it in enumerate(items):
        e = p.query(i)
        assert (e.bucket, e.slot) == (it["bucket"], it["slot"]), i
    for b, bk in enumerate(buckets):
        c = p.config(b)
        assert (c.path, c.padded_m, c.padded_n) == (0 if bk["path"] == "f32" else 1, bk["m_pad"], bk["n_pad"])
        assert (c.tile, c.algo, c.gram_restart, c.xcd_remap, c.apply_pass) == (
            bk["tile"], ALGO[bk["algo"]], bk["gram_restart"], bk["xcd_remap"], bk["apply_pass"]), b
        assert c.cost_ms_per_matrix == bk["cost"]
        assert p.bucket(b).tile == bk["tile"]


@pytest.mark.parametrize("bad", [_entry(1, 512, 768, tile=64), _entry(1, 128, 640, tile=256),
                                 _entry(1, 512, 768, tile=384), _entry(0, 256, 512, tile=128),
                                 _entry(0, 256, 512, algo=2), _entry(1, 512, 768, algo=3),
                                 _entry(1, 512, 768, restart=-1), _entry(1, 512, 768, remap=16),
                                 _entry(1, 512, 768, cost=-1.0), _entry(1, 512, 768, apply_pass=2),
                                 _entry(1, 512, 768, apply_pass=-1)])
def test_invalid_tuned_entries_rejected(bad):
    descs = CASES["mixed_odd"]
    with pytest.raises(ValueError):
        plan_reference(descs, tuned=[bad])
    with pytest.raises(d.DMuonError) as e:
        d.Plan(descs, tuning=_tune_entries([bad]))
    assert e.value.status == d.DMUON_ERR_INVALID_ARG
    # the same entry on a shape no bucket has is ignored
    d.Plan([(8, 8, 1, 1)], tuning=_tune_entries([bad])).close()


def test_tuning_cache_round_trip(tmp_path):
    path = str(tmp_path / "tune.json")
    assert d.load_tuning(path, key="devA") == []
    a = _tune_entries([_entry(1, 4096, 14336, tile=256, algo=2, restart=3, remap=4, cost=2.5),
                       _entry(1, 256, 1536, tile=128, algo=1, restart=1, remap=15, cost=0.25)])
    d.save_tuning(a, path, key="devA")
    d.save_tuning(_tune_entries([_entry(0, 64, 64, tile=64, algo=1, restart=1, remap=4, cost=0.01)]), path,
                  key="devB")
    # a later entry for the same shape replaces the earlier one
    d.save_tuning(_tune_entries([_entry(1, 256, 1536, tile=256, algo=2, restart=3, remap=0, cost=0.2)]), path,
                  key="devA")
    got = {(e.padded_m, e.padded_n): e.to_dict() for e in d.load_tuning(path, key="devA")}
    assert got[(4096, 14336)] == a[0].to_dict()
    assert got[(256, 1536)]["tile"] == 256 and got[(256, 1536)]["cost_ms_per_matrix"] == 0.2
    assert [e.padded_m for e in d.load_tuning(path, key="devB")] == [64]
    assert d.load_tuning(path, key="devC") == []


def test_autotune_argument_errors():
    need = ctypes.c_size_t()
    arr = (d.MatrixDesc * 1)(d.MatrixDesc(1024, 4096, 1, 1))
    assert LIB.muon_autotune_workspace_bytes(arr, 1, None, None) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_autotune_workspace_bytes(arr, 1, None, ctypes.byref(need)) == d.DMUON_OK
    # the trial plans include the Gram-space one, whose workspace is the largest
    assert need.value >= d.Plan([(1024, 4096, 1, 1)], "gram_space").workspace_bytes()
    # several buckets: the final whole-batch trials run every bucket at once
    multi = [(128, 128, 1, 1)] * 3 + [(128, 512, 1, 1)] * 4 + [(768, 256, 1, 1)] * 2 + [(96, 160, 0, 0)]
    marr = (d.MatrixDesc * len(multi))(*[d.MatrixDesc(*x) for x in multi])
    for algo in ("auto", "gram_space", "short_side"):
        opts = d._plan_opts(algo, 0, None)
        assert LIB.muon_autotune_workspace_bytes(marr, len(multi), ctypes.byref(opts),
                                                 ctypes.byref(need)) == d.DMUON_OK
        assert need.value >= d.Plan(multi, algo).workspace_bytes()
    got = ctypes.c_int32()
    res = (d.TuneEntry * 1)()
    for reps, cap in ((0, 1), (1, 0)):
        assert LIB.muon_autotune(arr, 1, None, _arr([8]), _arr([16]), 5, 3.4445, -4.775, 2.0315, reps, None, 0,
                                 None, res, cap, ctypes.byref(got)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_autotune(arr, 1, None, _arr([8]), _arr([16]), 5, 3.4445, -4.775, 2.0315, 1, None, 0,
                             None, res, 1, ctypes.byref(got)) == d.DMUON_ERR_WORKSPACE


def test_workspace_covers_operands():
    descs = CASES["mixed_odd"]
    items, buckets = plan_reference(descs)
    need = 0
    for bk in buckets:
        es = 2 if bk["path"] == "bf16" else 4
        cnt = len(bk["members"])
        need += cnt * es * (2 * bk["m_pad"] * bk["n_pad"] + 2 * bk["m_pad"] ** 2)
        if bk["algo"] == "gram_space":  # P_k, P_{k+1} and A_k Q_k
            need += cnt * es * 3 * bk["m_pad"] ** 2
    assert d.Plan(descs).workspace_bytes() >= need
    # forcing the short side needs no Gram-space arrays, forcing the Gram space more
    assert d.Plan(descs, "short_side").workspace_bytes() < d.Plan(descs, "gram_space").workspace_bytes()
    assert d.Plan(descs, "gram_space").workspace_bytes() > d.Plan(descs).workspace_bytes()
    assert d.Plan([]).workspace_bytes() == 0


def test_plan_errors():
    with pytest.raises(d.DMuonError) as e:
        d.Plan([(0, 5, 1, 1)])
    assert e.value.status == d.DMUON_ERR_INVALID_ARG
    with pytest.raises(d.DMuonError) as e:
        d.Plan([(5, 5, 3, 1)])
    assert e.value.status == d.DMUON_ERR_INVALID_ARG
    with pytest.raises(d.DMuonError) as e:
        d.Plan([(1 << 30, 5, 1, 1)])
    assert e.value.status == d.DMUON_ERR_UNSUPPORTED
    # bf16 gradients: the long side is limited to 2^27; fp32 gradients are not
    with pytest.raises(d.DMuonError) as e:
        d.Plan([(5, (1 << 27) + 1, 1, 1)])
    assert e.value.status == d.DMUON_ERR_UNSUPPORTED
    d.Plan([(5, 1 << 27, 1, 1)]).close()
    # a bucket whose B X launch would exceed 2^31 - 1 tiles (here 4096 x 2^19)
    with pytest.raises(d.DMuonError) as e:
        d.Plan([(256, 1 << 27, 1, 1)] * 4096)
    assert e.value.status == d.DMUON_ERR_UNSUPPORTED
    d.Plan([(256, 1 << 27, 1, 1)] * 4095).close()
    d.Plan([(5, (1 << 27) + 1, 0, 0)]).close()
    out = ctypes.c_void_p()
    assert LIB.muon_plan(None, 3, ctypes.byref(out)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan(None, -1, ctypes.byref(out)) == d.DMUON_ERR_INVALID_ARG
    arr = (d.MatrixDesc * 1)(d.MatrixDesc(8, 8, 1, 1))
    assert LIB.muon_plan_ex(arr, 1, ctypes.byref(d.PlanOpts(3, 0)), ctypes.byref(out)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_ex(arr, 1, ctypes.byref(d.PlanOpts(0, -1)), ctypes.byref(out)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_ex(arr, 1, None, ctypes.byref(out)) == d.DMUON_OK
    LIB.muon_plan_destroy(out)
    algo = ctypes.c_int32()
    assert LIB.muon_plan_bucket_algo(None, 0, ctypes.byref(algo), None) == d.DMUON_ERR_INVALID_ARG
    p = d.Plan([(8, 8, 1, 1)])
    assert LIB.muon_plan_bucket_algo(p.handle, 1, ctypes.byref(algo), None) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_bucket_algo(p.handle, 0, None, None) == d.DMUON_OK
    with pytest.raises(d.DMuonError):
        p.query(1)
    with pytest.raises(d.DMuonError):
        p.bucket(-1)
    LIB.muon_plan_destroy(None)  # no-op


def _arr(vals):
    a = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        a[i] = v
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))


@host_only
def test_step_argument_errors_before_device_work():
    # Every call below fails validation, which happens before any HIP call, so
    # the (never dereferenced) fake addresses are safe here without a GPU.
    p = d.Plan([(8, 16, 1, 1), (16, 8, 1, 1)])
    ws_bytes = p.workspace_bytes()
    hp = d.HParams(0.02, 0.95, 0.0, 1e-7, 3.4445, -4.775, 2.0315, 5, 1)
    g, m, w = _arr([0x10000, 0x20000]), _arr([0x30000, 0x40000]), _arr([0x50000, 0x60000])
    ws = ctypes.c_void_p(0x1000000)
    step = LIB.muon_step_batched
    assert step(None, g, m, w, ctypes.byref(hp), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert step(p.handle, g, m, w, None, ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert step(p.handle, None, m, w, ctypes.byref(hp), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert step(p.handle, g, None, w, ctypes.byref(hp), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    bad = _arr([0x10008, 0x20000])  # misaligned
    assert step(p.handle, bad, m, w, ctypes.byref(hp), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    alias = _arr([0x50000, 0x20000])  # grads[0] == params[0]
    assert step(p.handle, alias, m, w, ctypes.byref(hp), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert step(p.handle, g, _arr([0x10000, 0x40000]), w, ctypes.byref(hp), ws, ws_bytes,
                None) == d.DMUON_ERR_INVALID_ARG
    assert step(p.handle, g, m, w, ctypes.byref(hp), None, ws_bytes, None) == d.DMUON_ERR_WORKSPACE
    assert step(p.handle, g, m, w, ctypes.byref(hp), ws, ws_bytes - 1, None) == d.DMUON_ERR_WORKSPACE
    assert step(p.handle, g, m, w, ctypes.byref(hp), ctypes.c_void_p(0x1000010), ws_bytes,
                None) == d.DMUON_ERR_WORKSPACE
    hp_bad = d.HParams(0.02, 0.95, 0.0, 1e-7, 3.4445, -4.775, 2.0315, -1, 1)
    assert step(p.handle, g, m, w, ctypes.byref(hp_bad), ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    # Byte ranges, not just pointers: the 8 x 16 matrices are 256 B in bf16 (grads,
    # params) and 512 B in fp32 (momenta).  No written buffer may overlap another.
    inside = lambda base, off: base + off
    assert step(p.handle, g, m, _arr([0x50000, inside(0x50000, 128)]), ctypes.byref(hp), ws, ws_bytes,
                None) == d.DMUON_ERR_INVALID_ARG  # params[1] starts inside params[0]
    assert step(p.handle, _arr([inside(0x30000, 256), 0x20000]), m, w, ctypes.byref(hp), ws, ws_bytes,
                None) == d.DMUON_ERR_INVALID_ARG  # grads[0] inside momenta[0]
    assert step(p.handle, g, _arr([0x30000, inside(0x1000000, 64)]), w, ctypes.byref(hp), ws, ws_bytes,
                None) == d.DMUON_ERR_INVALID_ARG  # momenta[1] inside the workspace
    assert step(p.handle, _arr([0x1000000 - 128, 0x20000]), m, w, ctypes.byref(hp), ws, ws_bytes,
                None) == d.DMUON_ERR_INVALID_ARG  # grads[0] runs into the workspace
    ortho = LIB.ns_orthogonalize_batched
    assert ortho(p.handle, g, _arr([0x50000, inside(0x10000, 16)]), 5, 3.4445, -4.775, 2.0315, 1e-7, ws, ws_bytes,
                 None) == d.DMUON_ERR_INVALID_ARG  # outputs[1] inside inputs[0]
    assert ortho(p.handle, g, w, -1, 3.4445, -4.775, 2.0315, 1e-7, ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert ortho(p.handle, g, g, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, ws_bytes, None) == d.DMUON_ERR_INVALID_ARG
    assert ortho(p.handle, g, w, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, 16, None) == d.DMUON_ERR_WORKSPACE


@host_only
def test_adamw_argument_errors_before_device_work():
    # every call fails validation before any HIP call (fake addresses never dereferenced)
    n = (ctypes.c_int64 * 2)(100, 8)
    pd, gd = (ctypes.c_int32 * 2)(1, 0), (ctypes.c_int32 * 2)(1, 1)
    P, G = _arr([0x10000, 0x20000]), _arr([0x30000, 0x40000])
    M, V = _arr([0x50000, 0x60000]), _arr([0x70000, 0x80000])
    hp = d.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    f = LIB.adamw_step_batched
    E = d.DMUON_ERR_INVALID_ARG
    assert f(-1, n, pd, gd, P, G, M, V, ctypes.byref(hp), None) == E
    assert f(2, n, pd, gd, P, G, M, V, None, None) == E
    assert f(2, None, pd, gd, P, G, M, V, ctypes.byref(hp), None) == E
    assert f(2, n, pd, gd, P, None, M, V, ctypes.byref(hp), None) == E
    for bad in (d.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0), d.AdamWHParams(1e-3, 1.0, 0.999, 1e-8, 0.01, 1),
                d.AdamWHParams(1e-3, 0.9, -0.1, 1e-8, 0.01, 1), d.AdamWHParams(1e-3, 0.9, 0.999, 0.0, 0.01, 1),
                d.AdamWHParams(float("nan"), 0.9, 0.999, 1e-8, 0.01, 1)):
        assert f(2, n, pd, gd, P, G, M, V, ctypes.byref(bad), None) == E
    assert f(2, n, (ctypes.c_int32 * 2)(1, 7), gd, P, G, M, V, ctypes.byref(hp), None) == E
    assert f(2, (ctypes.c_int64 * 2)(100, -1), pd, gd, P, G, M, V, ctypes.byref(hp), None) == E
    assert f(2, n, pd, gd, _arr([0x10004, 0x20000]), G, M, V, ctypes.byref(hp), None) == E  # misaligned
    assert f(2, n, pd, gd, P, _arr([0x10000, 0x40000]), M, V, ctypes.byref(hp), None) == E  # g aliases p
    assert f(2, n, pd, gd, P, G, M, _arr([0x50000, 0x80000]), ctypes.byref(hp), None) == E  # v aliases m
    # byte ranges: tensor 0 holds 100 elements (200 B of bf16 params, 400 B of fp32 moments)
    assert f(2, n, pd, gd, P, G, _arr([0x50000, 0x50000 + 256]), V, ctypes.byref(hp), None) == E  # m[1] in m[0]
    assert f(2, n, pd, gd, P, _arr([0x10000 + 64, 0x40000]), M, V, ctypes.byref(hp), None) == E  # g[0] in p[0]
    # count 0 and all-empty tensors enqueue nothing
    assert f(0, None, None, None, None, None, None, None, ctypes.byref(hp), None) == d.DMUON_OK
    z = (ctypes.c_int64 * 2)(0, 0)
    assert f(2, z, pd, gd, _arr([0, 0]), _arr([0, 0]), _arr([0, 0]), _arr([0, 0]), ctypes.byref(hp),
             None) == d.DMUON_OK


def test_empty_plan_is_noop():
    p = d.Plan([])
    hp = d.HParams(0.02, 0.95, 0.0, 1e-7, 3.4445, -4.775, 2.0315, 5, 1)
    assert LIB.muon_step_batched(p.handle, None, None, None, ctypes.byref(hp), None, 0, None) == d.DMUON_OK
    assert LIB.ns_orthogonalize_batched(p.handle, None, None, 5, 3.4445, -4.775, 2.0315, 1e-7, None, 0,
                                        None) == d.DMUON_OK


def test_header_is_plain_c():
    # the boundary header compiles as C99 on its own (no HIP or torch types)
    import subprocess
    import tempfile

    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "t.c")
        with open(src, "w") as f:
            f.write('#include "dmuon_ns.h"\nint main(void){ dmuon_hparams h; (void)h; return 0; }\n')
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{inc}", src, "-o",
                            os.path.join(td, "t")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_program_links_and_plans():
    # a plain C99 program against the shared library: plan, query, workspace,
    # status strings and argument errors, no Python in between
    import subprocess
    import tempfile

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc, libdir = os.path.join(root, "include"), os.path.dirname(d.library_path())
    prog = r'''
#include <stdio.h>
#include "dmuon_ns.h"
int main(void) {
    dmuon_matrix_desc descs[3] = {{4096, 14336, DMUON_BF16, DMUON_BF16}, {14336, 4096, DMUON_BF16, DMUON_F32},
                                  {256, 512, DMUON_F32, DMUON_F32}};
    dmuon_plan* plan = NULL;
    if (muon_plan(descs, 3, &plan) != DMUON_OK) return 1;
    int32_t count = 0, buckets = 0, algo = 0, restart = 0, bucket = -1, slot = -1, tr = -1;
    size_t ws = 0;
    int64_t pm = 0, pn = 0, cost = 0;
    if (muon_plan_info(plan, &count, &buckets) != DMUON_OK || count != 3 || buckets != 2) return 2;
    if (muon_plan_workspace_bytes(plan, &ws) != DMUON_OK || ws == 0) return 3;
    if (muon_plan_query(plan, 1, &bucket, &slot, &tr, &pm, &pn, &cost) != DMUON_OK) return 4;
    if (bucket != 0 || slot != 1 || tr != 1 || pm != 4096 || pn != 14336) return 5;
    if (muon_plan_bucket_algo(plan, 0, &algo, &restart) != DMUON_OK || algo != DMUON_ALGO_GRAM_SPACE || restart != 3)
        return 6;
    if (muon_plan_query(plan, 3, &bucket, NULL, NULL, NULL, NULL, NULL) != DMUON_ERR_INVALID_ARG) return 7;
    dmuon_hparams hp = {0.02f, 0.95f, 0.0f, 1e-7f, 3.4445f, -4.7750f, 2.0315f, 5, 1};
    if (muon_step_batched(plan, NULL, NULL, NULL, &hp, NULL, 0, NULL) != DMUON_ERR_INVALID_ARG) return 8;
    muon_plan_destroy(plan);
    printf("%s %s\n", dmuon_version(), dmuon_status_string(DMUON_ERR_WORKSPACE));
    return 0;
}
'''
    with tempfile.TemporaryDirectory() as td:
        src, exe = os.path.join(td, "p.c"), os.path.join(td, "p")
        with open(src, "w") as f:
            f.write(prog)
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{inc}", src, f"-L{libdir}", "-ldmuon_ns",
                            f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
        assert r.stdout.split()[0] == d.version()


def test_binding_tensor_checks(monkeypatch):
    # the binding's per-call validation, on host tensors standing in for device
    # ones (the current device reported as -1, the index a host tensor gives)
    monkeypatch.setattr(torch.cuda, "current_device", lambda: -1)

    def on_current_device(t, what):
        if t.get_device() != torch.cuda.current_device():
            raise ValueError(f"{what} is on another device")

    monkeypatch.setattr(d, "_on_current_device", on_current_device)
    plan = d.Plan([(4, 8, 1, 0), (8, 4, 0, 1)])
    good = {"grad": [torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(8, 4)],
            "param": [torch.zeros(4, 8), torch.zeros(8, 4, dtype=torch.bfloat16)],
            "momentum": [torch.zeros(4, 8), torch.zeros(8, 4)]}
    for kind, ts in good.items():
        d._check_tensors(plan, ts, kind, kind)
    with pytest.raises(ValueError, match="expected 2 tensors"):
        d._check_tensors(plan, good["grad"][:1], "grads", "grad")
    with pytest.raises(ValueError, match=r"grads\[1\]: expected torch.float32"):
        d._check_tensors(plan, [good["grad"][0], torch.zeros(8, 4, dtype=torch.bfloat16)], "grads", "grad")
    with pytest.raises(ValueError, match=r"params\[0\]: expected contiguous 4x8"):
        d._check_tensors(plan, [torch.zeros(8, 4).t(), good["param"][1]], "params", "param")
    with pytest.raises(ValueError, match=r"momenta\[1\]: expected contiguous 8x4"):
        d._check_tensors(plan, [good["momentum"][0], torch.zeros(4, 8)], "momenta", "momentum")
    # a tensor on another device than the current one
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    with pytest.raises(ValueError, match=r"grads\[0\] is on another device"):
        d._check_tensors(plan, good["grad"], "grads", "grad")


def test_update_fused_by_hand():
    # with apply_pass 0: the resident kernel writes every member of a resident
    # bucket (any parameter type, any cols); the last B X launch writes a bf16
    # parameter's update when cols % 8 == 0 and its bucket runs tiled bf16
    # launches; ns_steps 0 has no iteration at all
    descs = [(1024, 4096, 1, 1), (4096, 1024, 1, 1), (520, 300, 1, 1), (384, 1000, 1, 0), (120, 256, 1, 1),
             (256, 512, 0, 0), (128, 640, 1, 1), (300, 520, 1, 1), (264, 136, 1, 1), (100, 250, 1, 0),
             (250, 100, 1, 0)]
    want = [True, True, False, False, True, False, True, True, True, True, True]
    p = d.Plan(descs)
    assert [p.bucket(p.query(i).bucket).resident for i in (4, 9, 10)] == [True] * 3
    assert not any(p.bucket(p.query(i).bucket).resident for i in (0, 2, 6, 8))
    assert [p.update_fused(i) for i in range(len(descs))] == want
    assert not any(p.update_fused(i, 0) for i in range(len(descs)))
    assert [p.update_fused(i, 1) for i in range(len(descs))] == want
    # apply_pass 1 on one bucket sends its members through the apply pass: the
    # 1024 x 4096 one (and its transpose), then the resident 128 x 256 one
    for i, members in ((0, (0, 1)), (9, (4, 9, 10))):
        e = p.config(p.query(i).bucket)
        e.apply_pass = 1
        q = d.Plan(descs, tuning=[e])
        assert [q.update_fused(k) for k in range(len(descs))] == [w and k not in members for k, w in enumerate(want)]
    # forced onto the Gram space, the 128 x 256 bucket is no longer resident: its
    # bf16 parameter with cols 256 stays fused, the others fall back to the apply pass
    g = d.Plan(descs, "gram_space")
    assert not g.bucket(g.query(4).bucket).resident
    assert [g.update_fused(i) for i in (4, 9, 10)] == [True, False, False]
    res = ctypes.c_int32()
    assert LIB.muon_plan_update_fused(None, 0, 5, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_update_fused(p.handle, len(descs), 5, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_update_fused(p.handle, -1, 5, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_update_fused(p.handle, 0, -1, ctypes.byref(res)) == d.DMUON_ERR_INVALID_ARG
    assert LIB.muon_plan_update_fused(p.handle, 0, 5, None) == d.DMUON_ERR_INVALID_ARG
