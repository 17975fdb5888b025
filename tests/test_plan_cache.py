"""Plan memoization (host only, no GPU): the cache returns the same plan for
an equal page table, builds a new one when the KV lengths change with the
same rows [FreeToken issue "Layer-major prefill for offloaded MoE": a plan
cache keyed by rows alone was wrong once split-KV depended on KV length],
when the parameters or page size change, and evicts least recently used
plans beyond its capacity. Plans from the cache equal freshly built ones
field by field and match the oracle planner."""
import numpy as np
import pytest

import paged_split_kv_v2_amd as pdk
import workloads as W
from oracle import planner as oplan

FIELDS = ("members", "group_indptr", "span_pages", "l0_indptr", "l0_indices", "l0_len",
          "l1_indptr", "l1_indices", "l1_len", "merge_indptr", "fused_merge_indptr",
          "group_of", "member_rank")


def table(seed=2100, suffix_max=300):
    b = W.cascade_shared_prefix(seed=seed, groups=3, members=5, prefix_tokens=1024,
                                suffix_max=suffix_max, extra=3, extra_tokens=700)
    return b.indptr.copy(), b.indices.copy(), b.kv_len.copy()


PARAMS = pdk.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=256,
                           l1_partition_tokens=512)


def same_plan(a, b):
    for f in FIELDS:
        assert np.array_equal(a.field(f), b.field(f)), f
    assert a.stats() == b.stats()


def test_hit_returns_the_same_plan_for_every_layer():
    cache = pdk.PlanCache(4)
    ip, ix, kl = table()
    first, hit = cache.get(ip, ix, kl, 16, PARAMS)
    assert not hit
    for layer in range(31):
        plan, hit = cache.get(ip.copy(), ix.copy(), kl.copy(), 16, PARAMS)
        assert hit and plan is first
    assert cache.stats() == {"lookups": 32, "hits": 31, "builds": 1, "evictions": 0,
                             "entries": 1}
    same_plan(first, pdk.CascadePlan(ip, ix, kl, 16, PARAMS))


def test_kv_length_change_is_a_miss():
    cache = pdk.PlanCache(4)
    ip, ix, kl = table()
    a, _ = cache.get(ip, ix, kl, 16, PARAMS)
    kl2 = kl.copy()
    kl2[0] -= 1                     # same rows, one token fewer
    assert (kl2[0] + 15) // 16 == (kl[0] + 15) // 16
    b, hit = cache.get(ip, ix, kl2, 16, PARAMS)
    assert not hit and b is not a
    same_plan(b, pdk.CascadePlan(ip, ix, kl2, 16, PARAMS))
    # the level-1 lengths differ, so a row-keyed cache would have been wrong
    assert not np.array_equal(a.field("l1_len"), b.field("l1_len"))


def test_parameters_and_page_size_are_part_of_the_key():
    cache = pdk.PlanCache(8)
    ip, ix, kl = table()
    cache.get(ip, ix, kl, 16, PARAMS)
    other = pdk.CascadeParams(enabled=1, max_groups=1, l0_partition_tokens=256,
                              l1_partition_tokens=512)
    _, hit = cache.get(ip, ix, kl, 16, other)
    assert not hit
    _, hit = cache.get(ip, ix, kl, 16,
                       pdk.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=256,
                                         l1_partition_tokens=512, fuse_levels=0))
    assert not hit
    # page size 8: the same ids and lengths are a different (valid) table
    kl8 = np.minimum(kl, 8 * np.diff(ip)).astype(np.int32)
    _, hit = cache.get(ip, ix, kl8, 8, pdk.CascadeParams(enabled=1, max_groups=0,
                                                         l0_partition_tokens=256,
                                                         l1_partition_tokens=512))
    assert not hit
    assert cache.stats()["builds"] == 4


def test_least_recently_used_plan_is_evicted():
    cache = pdk.PlanCache(2)
    t = [table(seed) for seed in (2101, 2102, 2103)]
    cache.get(*t[0], 16, PARAMS)
    cache.get(*t[1], 16, PARAMS)
    _, hit = cache.get(*t[0], 16, PARAMS)      # t0 most recent, t1 least
    assert hit
    cache.get(*t[2], 16, PARAMS)              # evicts t1
    _, hit = cache.get(*t[0], 16, PARAMS)
    assert hit
    _, hit = cache.get(*t[1], 16, PARAMS)
    assert not hit
    st = cache.stats()
    assert st["evictions"] == 2 and st["entries"] == 2 and st["builds"] == 4


def test_cached_plan_matches_the_oracle_planner():
    cache = pdk.PlanCache(2)
    ip, ix, kl = table(2104)
    plan, _ = cache.get(ip, ix, kl, 16, PARAMS)
    ref = oplan.build_cascade_plan(ip, ix, kl, 16, oplan.CascadeParams(
        enabled=1, max_groups=0, l0_partition_tokens=256, l1_partition_tokens=512))
    assert np.array_equal(plan.field("members"), np.asarray(ref.members, np.int32))
    assert np.array_equal(plan.field("l1_len"), np.asarray(ref.l1_len, np.int32))


def test_invalid_tables_are_rejected_and_not_cached():
    cache = pdk.PlanCache(2)
    with pytest.raises(pdk.PdkError):
        cache.get([0, 1], [3], [40], 16, PARAMS)   # 40 tokens need 3 pages
    with pytest.raises(pdk.PdkError):
        pdk.PlanCache(0)
    assert cache.stats()["entries"] == 0
