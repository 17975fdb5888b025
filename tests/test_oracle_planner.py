"""Pins for the oracle's shared-prefix planner (no GPU).

The page prints no plan values, so the planner is pinned by: a plan worked by
hand for the tiny workload (tests/golden/tiny_gqa_plan.json), brute force on
tiny batches (a different span search plus exhaustive selection), page-for-page
conservation between the two levels and the flat view, and one crafted batch
per rejection rule [cascade-PR, "Task items" item 4, "Correctness coverage"].
The readings R1-R8 in the planner module's docstring are this build's own
where the page is silent: those parts are pinned only by the brute force and
the hand-worked plan, not by values on the page.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import planner
from oracle.planner import CascadeParams
from workloads import tiny_gqa_fp32, cascade_shared_prefix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def csr(lists, lens):
    indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    indices = np.array([p for x in lists for p in x], np.int32)
    return indptr, indices, np.array(lens, np.int32)


def test_tiny_plan_matches_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "tiny_gqa_plan.json")))
    b = tiny_gqa_fp32()
    params = CascadeParams(**g["params"])
    plan = planner.build_cascade_plan(b.indptr, b.indices, b.kv_len, b.page_size, params)
    assert plan.decline == g["decline"]
    assert plan.members.tolist() == g["members"]
    assert plan.group_indptr.tolist() == g["group_indptr"]
    assert plan.span_pages.tolist() == g["span_pages"]
    assert plan.l0_len.tolist() == g["l0_len"]
    assert plan.l1_len.tolist() == g["l1_len"]
    assert np.diff(plan.l1_indptr).tolist() == g["l1_pages"]
    assert plan.merge_indptr.tolist() == g["merge_indptr"]
    assert plan.stats == g["stats"]
    assert plan.l0_indices.tolist() == b.indices[:2].tolist()


def conservation(plan, indptr, indices, kv_len, P):
    for b in range(len(kv_len)):
        flat = indices[indptr[b]:indptr[b + 1]].tolist()
        l1 = plan.l1_indices[plan.l1_indptr[b]:plan.l1_indptr[b + 1]].tolist()
        k = int(plan.group_of[b])
        if k >= 0:
            l0 = plan.l0_indices[plan.l0_indptr[k]:plan.l0_indptr[k + 1]].tolist()
            assert l0 + l1 == flat
            assert plan.l0_len[k] + plan.l1_len[b] == kv_len[b]
            assert plan.l1_len[b] >= 1
        else:
            assert l1 == flat and plan.l1_len[b] == kv_len[b]


def brute_span(mem, indptr, indices, kv_len, P):
    """Largest k such that every member has k full pages and all members
    hold the same ids at positions 0..k-1 (searched from the top down)."""
    kmax = min(int(kv_len[b]) // P for b in mem)
    for k in range(kmax, -1, -1):
        ok = all(indices[indptr[b]:indptr[b] + k].tolist() ==
                 indices[indptr[mem[0]]:indptr[mem[0]] + k].tolist() for b in mem)
        if ok:
            return k
    return 0


def brute_force_plan(indptr, indices, kv_len, P, params):
    B = len(kv_len)
    firsts = {}
    for b in range(B):
        if indptr[b + 1] > indptr[b]:
            firsts.setdefault(int(indices[indptr[b]]), []).append(b)
    groups = []
    for mem in firsts.values():
        if len(mem) < 2:
            continue
        span = brute_span(mem, indptr, indices, kv_len, P)
        npg = [int(indptr[b + 1] - indptr[b]) for b in mem]
        valid = (len(mem) >= params.min_members and span >= max(1, params.min_shared_pages)
                 and all(span < n for n in npg))
        groups.append((mem, span, valid))
    ok = [g for g in groups if g[2]]
    if not ok:
        return None, groups
    limit = len(ok) if params.max_groups == 0 else params.max_groups
    best, best_key = None, None
    for r in range(1, min(limit, len(ok)) + 1):
        for combo in itertools.combinations(ok, r):
            saved = sum(s * (len(m) - 1) for m, s, _ in combo)
            # prefer more saved reads, then the lexicographically smallest
            # sorted score/first-index list (the planner's tie-break)
            key = (saved, [(-s * (len(m) - 1), m[0]) for m, s, _ in
                           sorted(combo, key=lambda g: (-g[1] * (len(g[0]) - 1), g[0][0]))])
            if best is None or key[0] > best_key[0] or (key[0] == best_key[0] and key[1] < best_key[1]):
                best, best_key = combo, key
    return sorted(best, key=lambda g: g[0][0]), groups


@pytest.mark.parametrize("max_groups", [1, 0, 2])
def test_brute_force_on_tiny_batches(max_groups):
    rng = np.random.default_rng(100 + max_groups)
    P = 2
    n_checked = 0
    for trial in range(1500):
        B = int(rng.integers(1, 7))
        lists, lens = [], []
        for b in range(B):
            n = int(rng.integers(0, 7))
            # draw ids from a tiny alphabet so that prefixes collide often
            lists.append([int(x) for x in rng.choice([0, 1, 2, 3], size=n)])
        for b in range(B):
            npg = len(lists[b])
            lens.append(0 if npg == 0 else int(rng.integers((npg - 1) * P + 1, npg * P + 1)))
        indptr, indices, kv_len = csr(lists, lens)
        params = CascadeParams(enabled=1, min_shared_pages=int(rng.integers(1, 3)),
                               min_members=int(rng.integers(2, 4)), max_groups=max_groups,
                               l0_partition_tokens=2, l1_partition_tokens=4)
        plan = planner.build_cascade_plan(indptr, indices, kv_len, P, params)
        want, groups = brute_force_plan(indptr, indices, kv_len, P, params)
        if want is None:
            assert plan.groups == []
            assert plan.decline != "none"
        else:
            n_checked += 1
            assert [g.members for g in plan.groups] == [m for m, _, _ in want]
            assert [g.span_pages for g in plan.groups] == [s for _, s, _ in want]
        conservation(plan, indptr, indices, kv_len, P)
    assert n_checked > 100


def test_random_batches_conserve_pages():
    for seed in range(30):
        rng = np.random.default_rng(seed)
        B = int(rng.integers(2, 12))
        base = list(range(100, 100 + 20))
        lists, lens = [], []
        for b in range(B):
            k = int(rng.integers(0, 20))
            own = [1000 + 100 * b + j for j in range(int(rng.integers(1, 6)))]
            lists.append(base[:k] + own if rng.random() < 0.7 else own)
            lens.append(len(lists[-1]) * 4 - int(rng.integers(0, 4)))
        indptr, indices, kv_len = csr(lists, lens)
        for mg in (0, 1):
            plan = planner.build_cascade_plan(indptr, indices, kv_len, 4,
                                              CascadeParams(enabled=1, min_shared_pages=2,
                                                            max_groups=mg))
            conservation(plan, indptr, indices, kv_len, 4)


def test_disabled_and_default_decline():
    indptr, indices, kv_len = csr([[1, 2, 3], [1, 2, 4]], [48, 48])
    for en in (-1, 0):
        plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                          CascadeParams(enabled=en, min_shared_pages=1))
        assert plan.decline == "disabled" and plan.stats["members"] == 0
        assert plan.merge_indptr.tolist() == [0, 1, 2]
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.decline == "none" and plan.span_pages.tolist() == [2]


def test_no_candidate():
    indptr, indices, kv_len = csr([[1, 2], [3, 4], []], [32, 32, 0])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.decline == "no_candidate"


def test_span_below_threshold():
    indptr, indices, kv_len = csr([[1, 2, 3], [1, 2, 4]], [48, 48])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=3))
    assert plan.decline == "span_below_min"


def test_members_below_threshold():
    indptr, indices, kv_len = csr([[1, 2, 3], [1, 2, 4]], [48, 48])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1, min_members=3))
    assert plan.decline == "members_below_min"


def test_span_reaching_a_last_page_falls_back():
    # request 1's whole (page-aligned) range is the shared prefix
    indptr, indices, kv_len = csr([[1, 2, 3], [1, 2]], [48, 32])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.decline == "reaches_last_page" and plan.groups == []


def test_partial_shared_page_is_not_shared():
    # page 2 is the (partly filled) last page of request 1: the full-page cap
    # keeps it out of the span, leaving one shared page
    indptr, indices, kv_len = csr([[1, 2, 3], [1, 2]], [48, 20])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.decline == "none" and plan.span_pages.tolist() == [1]
    assert plan.l1_len.tolist() == [32, 4]


def test_early_divergence_shortens_span_for_everyone():
    lists = [[1, 2, 3, 4, 9], [1, 2, 3, 4, 8], [1, 2, 7, 7, 7]]
    indptr, indices, kv_len = csr(lists, [80, 80, 80])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.members.tolist() == [0, 1, 2] and plan.span_pages.tolist() == [2]


def test_selection_by_saved_reads_and_tie_break():
    # group A: 3 members x 2 pages -> score 4; group B: 2 members x 4 pages -> 4;
    # tie -> lowest first batch index wins (B sits at slot 0)
    lists = [[5, 6, 7, 8, 50], [1, 2, 10], [5, 6, 7, 8, 51], [1, 2, 11], [1, 2, 12]]
    indptr, indices, kv_len = csr(lists, [80, 48, 80, 48, 48])
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1))
    assert plan.members.tolist() == [0, 2]
    plan = planner.build_cascade_plan(indptr, indices, kv_len, 16,
                                      CascadeParams(enabled=1, min_shared_pages=1, max_groups=0))
    assert plan.members.tolist() == [0, 2, 1, 3, 4]
    assert plan.group_indptr.tolist() == [0, 2, 5]
    assert plan.merge_indptr.tolist() == [0, 2, 4, 6, 8, 10]


def test_kill_switch_parse():
    for v in ("0", "false", "OFF", " no ", "False"):
        assert planner.enabled_from_env(v) == 0
    for v in ("1", "true", "On", "YES", " yes"):
        assert planner.enabled_from_env(v) == 1
    for v in (None, "", "2", "maybe", "enable"):
        assert planner.enabled_from_env(v) == -1


def test_stacked_head_map_is_kv_head_major():
    M, Hkv, G = 3, 2, 4
    Hq = Hkv * G
    hmap = planner.stacked_head_map(M, Hkv, G)
    assert sorted(hmap.tolist()) == list(range(M * Hq))       # a permutation
    for h0, target in enumerate(hmap):
        m, i = divmod(int(target), Hq)
        # the kernel reads KV head h0 // (M*G); the member's head reads i // G
        assert h0 // (M * G) == i // G
    # the [M, Hkv, G] -> [Hkv, M, G] transpose, spelled with numpy
    want = np.arange(M * Hq).reshape(M, Hkv, G).transpose(1, 0, 2).reshape(-1)
    assert np.array_equal(hmap, want)
    # member-major reads the wrong KV head for some heads
    mm = planner.member_major_head_map(M, Hkv, G)
    assert any(h0 // (M * G) != (int(t) % Hq) // G for h0, t in enumerate(mm))


def test_cascade_workload_plan():
    b = cascade_shared_prefix(groups=4, members=3, prefix_tokens=256, suffix_max=100,
                              extra=2, extra_tokens=64)
    plan = planner.build_cascade_plan(b.indptr, b.indices, b.kv_len, 16,
                                      CascadeParams(enabled=1, max_groups=0))
    assert plan.decline == "none" and len(plan.groups) == 4
    assert plan.span_pages.tolist() == [16] * 4
    gos = b.meta["group_of_slot"]
    for g in plan.groups:
        assert len({gos[m] for m in g.members}) == 1 and len(g.members) == 3
    conservation(plan, b.indptr, b.indices, b.kv_len, 16)
    one = planner.build_cascade_plan(b.indptr, b.indices, b.kv_len, 16,
                                     CascadeParams(enabled=1, max_groups=1))
    assert len(one.groups) == 1 and one.groups[0].members == plan.groups[0].members
