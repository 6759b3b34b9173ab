"""Pins of the planning rule's reference (oracle/plan_oracle.py) on hand-worked
examples, and of the Llama-3.1-8B owner share used as the headline workload."""

from collections import Counter

from matrix_optimizer_02_amd.workloads import (dense_ns_cost, get_workload, llama8b_full_set,
                                                lpt_bins)
from oracle import plan_reference

F32, BF16 = 0, 1


def test_small_batch_buckets_by_hand():
    # 32 x 128x128, 32 x 128x512, 32 x 512x128 (bf16): two buckets.
    # 128x512 bucket: 64 members x (4*128^2*512 + 2*128^3) = 64 x 37748736
    # 128x128 bucket: 32 members x 6*128^3 = 32 x 12582912 -> ordered second.
    descs = [(128, 128, BF16, BF16)] * 32 + [(128, 512, BF16, BF16)] * 32 + [(512, 128, BF16, BF16)] * 32
    items, buckets = plan_reference(descs)
    assert [(b["path"], b["m_pad"], b["n_pad"], len(b["members"])) for b in buckets] == [
        ("bf16", 128, 512, 64), ("bf16", 128, 128, 32)]
    assert buckets[0]["members"] == list(range(32, 96))
    assert items[0]["bucket"] == 1 and items[0]["slot"] == 0 and not items[0]["transposed"]
    assert items[40]["bucket"] == 0 and items[40]["slot"] == 8 and not items[40]["transposed"]
    assert items[70]["bucket"] == 0 and items[70]["slot"] == 38 and items[70]["transposed"]
    assert items[70]["cost"] == 37748736


def test_padding_and_paths_by_hand():
    descs = [(300, 700, BF16, BF16),   # m=300 -> g=256: 512 x 768
             (700, 300, BF16, F32),    # same bucket, transposed
             (100, 130, BF16, BF16),   # m=100 -> g=128: 128 x 256
             (256, 512, F32, F32),     # f32 path, g=64: 256 x 512
             (65, 65, F32, BF16)]      # f32: 128 x 128
    items, buckets = plan_reference(descs)
    keys = [(b["path"], b["m_pad"], b["n_pad"]) for b in buckets]
    # executed costs: 2 x (4*512^2*768 + 2*512^3) = 2 x 1073741824
    #                 4*256^2*512 + 2*256^3 = 167772160 ; 4*128^2*256+2*128^3 = 20971520 ;
    #                 6*128^3 = 12582912
    assert keys == [("bf16", 512, 768), ("f32", 256, 512), ("bf16", 128, 256), ("f32", 128, 128)]
    assert items[1]["transposed"] and items[1]["bucket"] == 0 and items[1]["slot"] == 1
    assert items[2]["m_pad"] == 128 and items[2]["n_pad"] == 256
    assert items[4]["m_pad"] == 128 and items[4]["bucket"] == 3
    assert not items[4]["transposed"]


def test_tie_keeps_first_appearance():
    descs = [(64, 64, F32, F32), (128, 128, BF16, BF16), (64, 64, F32, F32)]
    # f32 64x64 x2: 2*6*64^3 = 3145728 ; bf16 128x128: 6*128^3 = 12582912
    items, buckets = plan_reference(descs)
    assert [b["m_pad"] for b in buckets] == [128, 64]
    descs = [(128, 128, BF16, BF16), (128, 128, F32, F32)]  # f32 128 -> g=64 -> 128x128, equal cost
    items, buckets = plan_reference(descs)
    assert [b["path"] for b in buckets] == ["bf16", "f32"]


def test_llama8b_owner_share():
    full = llama8b_full_set()
    costs = [dense_ns_cost(s.rows, s.cols) for s in full]
    bins = lpt_bins(costs, 8)
    loads = {sum(costs[i] for i in b) for b in bins}
    assert len(loads) == 1  # perfectly balanced: 8 x 16647.293239296 GF per iteration
    assert loads.pop() == 16647293239296
    w = get_workload("llama3.1-8b_owner_1of8")
    assert w.count == 28
    assert Counter((s.rows, s.cols) for s in w.matrices) == Counter(
        {(4096, 4096): 8, (1024, 4096): 8, (14336, 4096): 8, (4096, 14336): 4})
    items, buckets = plan_reference([(s.rows, s.cols, BF16, BF16) for s in w.matrices])
    assert [(b["m_pad"], b["n_pad"], len(b["members"])) for b in buckets] == [
        (4096, 14336, 12), (4096, 4096, 8), (1024, 4096, 8)]


def test_recurrence_form_by_hand():
    # Default rule: Gram space for bf16 buckets with n_pad > m_pad, m_pad >= 1024 and every member n >= 3 m.
    # (300, 700): m_pad 512 < 1024 -> short side
    # (1024, 4096): m_pad 1024, 4096 >= 3*1024 -> Gram space, restart 2 (m_pad <= 1024)
    # (3400, 1100): m 1100 -> m_pad 1280, n 3400 -> n_pad 3584, 3400 >= 3300 -> Gram space, restart 3
    # (1100, 3200): m_pad 1280, n_pad 3328, 3200 < 3300 -> short side
    # (768, 3072): m_pad 768 < 1024 -> short side
    # (384, 500): m_pad 512 = n_pad 512 -> short side
    # (130, 600) f32: always short side (g = 64: 192 x 640)
    descs = [(300, 700, BF16, BF16), (1024, 4096, BF16, BF16), (3400, 1100, BF16, BF16), (1100, 3200, BF16, BF16),
             (768, 3072, BF16, BF16), (384, 500, BF16, BF16), (130, 600, F32, F32)]
    _, buckets = plan_reference(descs)
    form = {(b["path"], b["m_pad"], b["n_pad"]): (b["algo"], b["gram_restart"]) for b in buckets}
    assert form == {("bf16", 512, 768): ("short_side", 1), ("bf16", 1024, 4096): ("gram_space", 2),
                    ("bf16", 1280, 3584): ("gram_space", 3), ("bf16", 1280, 3328): ("short_side", 1),
                    ("bf16", 768, 3072): ("short_side", 1), ("bf16", 512, 512): ("short_side", 1),
                    ("f32", 192, 640): ("short_side", 1)}
    _, forced = plan_reference(descs, "gram_space", 2)
    assert {(b["path"], b["algo"], b["gram_restart"]) for b in forced} == {
        ("bf16", "gram_space", 2), ("f32", "short_side", 1)}
    # one member with n < 3 m keeps its whole bucket on the short side:
    # (1100, 3400) and (1150, 3400) both pad to 1280 x 3584; 3400 < 3 * 1150
    _, mixed = plan_reference([(1100, 3400, BF16, BF16), (1150, 3400, BF16, BF16)])
    assert [(b["m_pad"], b["n_pad"], b["algo"]) for b in mixed] == [(1280, 3584, "short_side")]


def test_tuned_entries_by_hand():
    descs = [(256, 512, BF16, BF16), (1024, 4096, BF16, BF16), (256, 512, BF16, BF16), (128, 128, BF16, BF16)]
    # dense order without measurements: 1024x4096 (1 x 19327352832), 256x512 (2 x 301989888),
    # 128x128 (1 x 12582912)
    _, b0 = plan_reference(descs)
    assert [(b["m_pad"], b["n_pad"]) for b in b0] == [(1024, 4096), (256, 512), (128, 128)]
    e = lambda mp, np_, **kw: {"path": BF16, "padded_m": mp, "padded_n": np_, **kw}
    tuned = [e(256, 512, tile=128, algo=1, xcd_remap=15, cost_ms_per_matrix=3.0),
             e(1024, 4096, algo=2, gram_restart=2, cost_ms_per_matrix=5.0),
             e(128, 128, cost_ms_per_matrix=6.0)]
    # measured order: 256x512 2 x 3.0 = 6.0 ties 128x128 1 x 6.0 (first appearance wins), then 5.0
    _, b1 = plan_reference(descs, tuned=tuned)
    assert [(b["m_pad"], b["tile"], b["algo"], b["gram_restart"], b["xcd_remap"]) for b in b1] == [
        (256, 128, "short_side", 1, 15), (128, 128, "short_side", 1, 4), (1024, 256, "gram_space", 2, 4)]
    # one bucket without a cost: the dense order stays
    _, b2 = plan_reference(descs, tuned=tuned[:2])
    assert [b["m_pad"] for b in b2] == [1024, 256, 128]
    # Entries are keyed by padded dims: under the default option an entry's Gram space
    # applies only where the default rule would take it on the bucket's real members.
    # (1100, 3400) and (1150, 3400) pad alike (1280 x 3584); only the first has n >= 3 m.
    g = [e(1280, 3584, algo=2, gram_restart=2)]
    _, ok = plan_reference([(1100, 3400, BF16, BF16)], tuned=g)
    _, refused = plan_reference([(1150, 3400, BF16, BF16)], tuned=g)
    _, forced = plan_reference([(1150, 3400, BF16, BF16)], "gram_space", tuned=g)
    assert [(b["algo"], b["gram_restart"]) for b in ok] == [("gram_space", 2)]
    assert [(b["algo"], b["gram_restart"]) for b in refused] == [("short_side", 1)]
    assert [(b["algo"], b["gram_restart"]) for b in forced] == [("gram_space", 2)]
    # the same for an entry on a bucket whose padded short side is under 1024
    _, small = plan_reference([(256, 1536, BF16, BF16)], tuned=[e(256, 1536, algo=2)])
    assert [b["algo"] for b in small] == ["short_side"]
