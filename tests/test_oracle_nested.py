"""Pins for the oracle's nested shared prefixes (no GPU).

What pins what:
  * a plan worked out by hand from the readings (tests/golden/nested_plan.json)
    at depths 1 and 3;
  * depth 1 is exactly the two-level plan of planner.py;
  * page conservation: a request's spans (read from their first member's
    page list) followed by its private pages are its own page list;
  * an independent check of the rules on random tables: members agree on a
    span's pages, a span cannot grow by one page under the full-page cap and
    the last-page rule, and a span's children are exactly the qualifying
    subgroups, recomputed here without the oracle's code;
  * the invariant the nested split rests on [cascade-PR, "How the #898 merge
    kernel is reused": merging is associative]: the nested composition equals
    flat attention, at every depth.
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention, nested, planner

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nested_plan.json")


def golden_batch():
    g = json.load(open(GOLDEN))
    names = sorted({p for pl in g["pages"] for p in pl})
    ids = {n: i for i, n in enumerate(names)}
    lists = [[ids[p] for p in pl] for pl in g["pages"]]
    b = W.paged_batch_from_lists("nested_golden", np.random.default_rng(2400), lists,
                                 g["kv_len"], page_size=g["page_size"], num_q_heads=4,
                                 num_kv_heads=2, head_dim_k=16, head_dim_v=16, kv_dtype="f32",
                                 q_dtype="f32", partition_tokens=8)
    return g, b


PARAMS = planner.CascadeParams(enabled=1, min_shared_pages=1, min_members=2, max_groups=0,
                               l0_partition_tokens=8, l1_partition_tokens=8)


@pytest.mark.parametrize("depth", [1, 3])
def test_hand_worked_plan(depth):
    g, b = golden_batch()
    want = g[f"depth{depth}"]
    plan = nested.build_nested_plan(b.indptr, b.indices, b.kv_len, b.page_size, PARAMS, depth)
    got = [dict(members=s.members, start_page=s.start_page, span_pages=s.span_pages,
                depth=s.depth, parent=s.parent) for s in plan.spans]
    assert got == want["spans"]
    assert plan.private_start_page.tolist() == want["private_start_page"]
    assert plan.merge_indptr.tolist() == want["merge_indptr"]


def test_depth_one_is_the_two_level_plan():
    for seed in range(2410, 2416):
        b = W.nested_shared_prefix(seed=seed, tenants=3, members=3, system_tokens=64,
                                   tenant_tokens=48, suffix_min=1, suffix_max=40, extra=2,
                                   extra_tokens=50, page_size=8)
        p = planner.CascadeParams(enabled=1, min_shared_pages=1, max_groups=0)
        two = planner.build_cascade_plan(b.indptr, b.indices, b.kv_len, b.page_size, p)
        one = nested.build_nested_plan(b.indptr, b.indices, b.kv_len, b.page_size, p, 1)
        assert [(s.members, s.span_pages) for s in one.spans] == \
            [(g.members, g.span_pages) for g in two.groups]
        assert all(s.start_page == 0 for s in one.spans)
        assert np.array_equal(one.merge_indptr, two.merge_indptr)


def random_nested_table(rng, P=4):
    """A random forest of shared pages: requests walk down a random tree of
    page runs, then take private pages (no oracle code involved)."""
    lists, nxt = [], 1000
    def run(n):
        nonlocal nxt
        r = list(range(nxt, nxt + n))
        nxt += n
        return r
    roots = [run(int(rng.integers(1, 4))) for _ in range(2)]
    kids = {i: [run(int(rng.integers(1, 3))) for _ in range(int(rng.integers(1, 3)))]
            for i in range(2)}
    for _ in range(int(rng.integers(4, 9))):
        i = int(rng.integers(0, 2))
        pl = list(roots[i])
        if rng.random() < 0.8:
            pl += kids[i][int(rng.integers(0, len(kids[i])))]
        pl += run(int(rng.integers(1, 3)))
        lists.append(pl)
    kv = [len(pl) * P - int(rng.integers(0, P)) for pl in lists]
    return lists, kv


def check_rules(lists, kv, P, plan, params, max_depth):
    pages = [len(pl) for pl in lists]
    for i, sp in enumerate(plan.spans):
        e = sp.start_page + sp.span_pages
        lead = lists[sp.members[0]]
        for b in sp.members:    # members agree on the span
            assert lists[b][sp.start_page:e] == lead[sp.start_page:e]
            assert e <= kv[b] // P and e < pages[b]
        # cannot grow by one page
        grows = all(e < pages[b] and e + 1 <= kv[b] // P and e + 1 < pages[b] and
                    lists[b][e] == lead[e] for b in sp.members)
        assert not grows
        # children are exactly the qualifying subgroups at position e
        if sp.depth + 1 < max_depth:
            groups = {}
            for b in sp.members:
                if pages[b] > e:
                    groups.setdefault(lists[b][e], []).append(b)
            want = []
            for mem in groups.values():
                if len(mem) < 2:
                    continue
                c = 0
                while all(e + c < pages[b] and lists[b][e + c] == lists[mem[0]][e + c]
                          for b in mem):
                    c += 1
                c = min([c] + [kv[b] // P - e for b in mem])
                if c >= 1 and all(e + c < pages[b] for b in mem):
                    want.append((sorted(mem), e, c))
            got = [(s.members, s.start_page, s.span_pages) for s in plan.spans
                   if s.parent == i]
            assert sorted(got) == sorted(want)


@pytest.mark.parametrize("max_depth", [2, 3, 4])
def test_random_tables_follow_the_rules_and_conserve_pages(max_depth):
    rng = np.random.default_rng(2420 + max_depth)
    P = 4
    params = planner.CascadeParams(enabled=1, min_shared_pages=1, min_members=2, max_groups=0)
    for trial in range(40):
        lists, kv = random_nested_table(rng, P)
        indptr = np.cumsum([0] + [len(pl) for pl in lists]).astype(np.int32)
        indices = np.asarray([p for pl in lists for p in pl], np.int32)
        plan = nested.build_nested_plan(indptr, indices, kv, P, params, max_depth)
        check_rules(lists, kv, P, plan, params, max_depth)
        for b, pl in enumerate(lists):
            rebuilt = []
            for i in plan.spans_of[b]:
                sp = plan.spans[i]
                rebuilt += lists[sp.members[0]][sp.start_page:sp.start_page + sp.span_pages]
            rebuilt += pl[int(plan.private_start_page[b]):]
            assert rebuilt == pl


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_nested_composition_equals_flat(depth):
    g, b = golden_batch()
    out, lse = nested.nested_cascade_decode(b, PARAMS, depth)
    fo, fl = attention.decode_attention(b)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12
    w = W.nested_shared_prefix(seed=2430, tenants=2, members=3, system_tokens=64,
                               tenant_tokens=32, suffix_min=1, suffix_max=40, extra=2,
                               extra_tokens=30, page_size=8)
    p = planner.CascadeParams(enabled=1, min_shared_pages=1, max_groups=0)
    out, lse, plan = nested.nested_cascade_decode(w, p, depth, return_plan=True)
    assert len(plan.spans) == (1 if depth == 1 else 3)
    fo, fl = attention.decode_attention(w)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12
