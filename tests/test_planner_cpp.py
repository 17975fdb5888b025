"""The library's C++ cascade planner against the oracle planner, bit for bit
(no GPU): every plan field, the stats and the decline reason, on the named
workloads, on seeded random page tables and on crafted rejection cases."""
import numpy as np
import pytest

import paged_split_kv_v2_amd as pdk
from oracle import planner as oplan
from plan_expect import fused_rows, nested_expected
from workloads import cascade_shared_prefix, tiny_gqa_fp32

FIELDS = ["members", "group_indptr", "span_pages", "l0_indptr", "l0_indices", "l0_len",
          "l1_indptr", "l1_indices", "l1_len", "merge_indptr", "group_of", "member_rank"]


def test_fused_rows_with_an_empty_level1_range():
    """Worked by hand: the tiny workload's batch (requests 0-2 share two
    pages and own 1/2/3 private pages, request 3 owns 4 pages, page 16) plus
    a fifth request of length 0, partitions of 32 tokens. Members own one
    level-0 row each (32 shared tokens) and 1/1/2 level-1 rows (16/32/48
    tokens); request 3 owns 2 level-1 rows; request 4's empty range owns one
    row."""
    b = tiny_gqa_fp32()
    indptr = np.concatenate([b.indptr, b.indptr[-1:]]).astype(np.int32)
    kv_len = np.concatenate([b.kv_len, [0]]).astype(np.int32)
    kw = dict(enabled=1, min_shared_pages=2, l0_partition_tokens=32, l1_partition_tokens=32)
    plan, ref = compare(indptr, b.indices, kv_len, 16, **kw)
    assert ref.l1_len.tolist() == [16, 32, 48, 64, 0]
    assert plan.field("fused_merge_indptr").tolist() == [0, 2, 4, 7, 9, 10]
    assert plan.field("merge_indptr").tolist() == [0, 2, 4, 6, 7, 8]


def compare(indptr, indices, kv_len, P, **kw):
    op = oplan.CascadeParams(**kw)
    ref = oplan.build_cascade_plan(indptr, indices, kv_len, P, op)
    plan = pdk.CascadePlan(indptr, indices, kv_len, P, pdk.CascadeParams(**kw))
    for f in FIELDS:
        want = np.asarray(getattr(ref, f), dtype=np.int64)
        got = plan.field(f).astype(np.int64)
        assert np.array_equal(got, want), f
    assert np.array_equal(plan.field("fused_merge_indptr"),
                          fused_rows(ref.group_of, ref.l0_len, ref.l1_len, op))
    stats, decline = plan.stats()
    assert stats == ref.stats
    assert decline == ref.decline
    return plan, ref


def test_tiny_workload_plan():
    b = tiny_gqa_fp32()
    plan, ref = compare(b.indptr, b.indices, b.kv_len, 16, enabled=1, min_shared_pages=2,
                        l0_partition_tokens=32, l1_partition_tokens=32)
    assert plan.stats()[0]["members"] == 3


@pytest.mark.parametrize("max_groups", [1, 0])
def test_cascade_workload_plan(max_groups):
    b = cascade_shared_prefix(poison=False)
    plan, ref = compare(b.indptr, b.indices, b.kv_len, 16, enabled=1, max_groups=max_groups,
                        l0_partition_tokens=256, l1_partition_tokens=512)
    assert len(ref.groups) == (4 if max_groups == 0 else 1)


def test_random_page_tables():
    n = 0
    for seed in range(1000):
        rng = np.random.default_rng(seed)
        B = int(rng.integers(1, 10))
        P = int(rng.choice([1, 2, 4, 16]))
        lists, lens = [], []
        for b in range(B):
            npg = int(rng.integers(0, 8))
            lists.append([int(x) for x in rng.choice(6, size=npg)])
            lens.append(0 if npg == 0 else int(rng.integers((npg - 1) * P + 1, npg * P + 1)))
        indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
        indices = np.array([p for x in lists for p in x], np.int32)
        kw = dict(enabled=int(rng.choice([-1, 0, 1, 1, 1])),
                  min_shared_pages=int(rng.integers(1, 4)), min_members=int(rng.integers(2, 4)),
                  max_groups=int(rng.integers(0, 3)), l0_partition_tokens=P * int(rng.integers(1, 4)),
                  l1_partition_tokens=P * int(rng.integers(1, 4)))
        plan, ref = compare(indptr, indices, np.array(lens, np.int32), P, **kw)
        n += ref.decline == "none"
    assert n > 60


@pytest.mark.parametrize("lists,lens,kw,reason", [
    ([[1, 2, 3], [1, 2, 4]], [48, 48], dict(enabled=-1), "disabled"),
    ([[1, 2, 3], [1, 2, 4]], [48, 48], dict(enabled=0), "disabled"),
    ([[1, 2], [3, 4]], [32, 32], dict(enabled=1, min_shared_pages=1), "no_candidate"),
    ([[1, 2, 3], [1, 2, 4]], [48, 48], dict(enabled=1, min_shared_pages=3), "span_below_min"),
    ([[1, 2, 3], [1, 2, 4]], [48, 48], dict(enabled=1, min_shared_pages=1, min_members=3),
     "members_below_min"),
    ([[1, 2, 3], [1, 2]], [48, 32], dict(enabled=1, min_shared_pages=1), "reaches_last_page"),
    ([[1, 2, 3], [1, 2]], [48, 20], dict(enabled=1, min_shared_pages=1), "none"),
])
def test_rejections(lists, lens, kw, reason):
    indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    indices = np.array([p for x in lists for p in x], np.int32)
    plan, ref = compare(indptr, indices, np.array(lens, np.int32), 16, **kw)
    assert plan.stats()[1] == reason


def test_invalid_plan_arguments():
    with pytest.raises(pdk.PdkError):
        pdk.CascadePlan([0, 1], [3], [40], 16, pdk.CascadeParams(enabled=1))  # 1 page, 40 tokens
    with pytest.raises(pdk.PdkError):
        pdk.CascadePlan([0, 1], [3], [16], 16, pdk.CascadeParams(enabled=1, min_members=1))
    with pytest.raises(pdk.PdkError):
        pdk.CascadePlan([0, 1], [3], [16], 16,
                        pdk.CascadeParams(enabled=1, l1_partition_tokens=24))


@pytest.mark.parametrize("depth", [2, 3])
def test_nested_plans_match_the_oracle(depth):
    from workloads import nested_shared_prefix
    cases = []
    for seed in range(2500, 2504):
        b = nested_shared_prefix(seed=seed, tenants=3, members=4, system_tokens=64,
                                 tenant_tokens=48, suffix_min=1, suffix_max=40, extra=2,
                                 extra_tokens=50, page_size=8, poison=False)
        cases.append((b.indptr, b.indices, b.kv_len, 8))
    b = nested_shared_prefix(poison=False)
    cases.append((b.indptr, b.indices, b.kv_len, 16))
    for indptr, indices, kv_len, P in cases:
        kw = dict(enabled=1, min_shared_pages=1, max_groups=0, l0_partition_tokens=4 * P,
                  l1_partition_tokens=8 * P)
        ref, want = nested_expected(indptr, indices, kv_len, P, oplan.CascadeParams(**kw), depth)
        assert sum(s.depth > 0 for s in ref.spans) > 0
        plan = pdk.CascadePlan(indptr, indices, kv_len, P, pdk.CascadeParams(max_depth=depth, **kw))
        for f, v in want.items():
            assert np.array_equal(plan.field(f).astype(np.int64), np.asarray(v, np.int64)), f
        # single-merge layout: every span holding the request, then its
        # level-1 rows (at least one)
        S0, S1 = kw["l0_partition_tokens"], kw["l1_partition_tokens"]
        rows = [0]
        for b, n1 in enumerate(want["l1_len"]):
            n0 = sum(-(-ref.spans[k].span_pages * P // S0) for k in ref.spans_of[b])
            rows.append(rows[-1] + n0 + max(1, -(-int(n1) // S1)))
        assert plan.field("fused_merge_indptr").tolist() == rows
        stats, decline = plan.stats()
        S0, S1 = kw["l0_partition_tokens"], kw["l1_partition_tokens"]
        assert decline == ref.decline
        assert stats["members"] == sum(1 for s in ref.spans_of if s)
        assert stats["shared_pages"] == sum(s.span_pages for s in ref.spans)
        assert stats["prefix_chunks"] == sum(-(-s.span_pages * P // S0) for s in ref.spans)
        assert stats["suffix_chunks"] == sum(-(-int(n) // S1) for n in want["l1_len"])


def test_max_depth_is_validated():
    b = tiny_gqa_fp32()
    with pytest.raises(pdk.PdkError):
        pdk.CascadePlan(b.indptr, b.indices, b.kv_len, 16, pdk.CascadeParams(enabled=1, max_depth=0))
