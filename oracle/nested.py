"""Nested shared prefixes: spans inside spans (a system prompt shared by all
requests, a sub-prefix shared by each tenant's requests, private suffixes).

Test infrastructure only. [cascade-PR, "What I left out, and where I was
unsure"] scopes nested sharing out ("a common system prompt plus a
per-tenant sub-prefix would need a third level"); [cascade-PR, "How the #898
merge kernel is reused"] makes the merge side follow: merging is associative,
so the states of any split of a request's range into disjoint pieces merge
to the flat state. The decomposition below is this package's reading, built
on the two-level rules of planner.py:

  N1 The outermost spans are the two-level planner's selection (grouping by
     first page, common prefix, full-page cap, last-page rule, thresholds,
     score, max_groups).
  N2 Below a span covering pages [s, e) of members M, the members that have
     a page at position e are grouped by that page id; a subgroup becomes a
     child span [e, e + c) when it has at least min_members members and its
     positional common prefix from e, capped so that every shared page is
     full (c <= kv_len // P - e for each member), is at least
     min_shared_pages pages and ends before every member's last page
     (e + c < page count). A subgroup that fails a check keeps those pages
     private.
  N3 Every qualifying subgroup of a span becomes a child (they are disjoint);
     children are ordered by first member, and the recursion stops at
     max_depth levels of spans (max_depth = 1 is the two-level plan).
  N4 Spans are numbered level by level (all outermost spans by first member,
     then all second-level spans by first member, ...).
  N5 A request's private range starts at the end of the deepest span that
     holds it. Its merge group has one row per span holding it (outermost
     first) and one for the private range.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from . import attention, planner
from .codecs import decode


@dataclass
class Span:
    members: List[int]
    start_page: int
    span_pages: int
    depth: int           # 0 = outermost
    parent: int          # index of the enclosing span, -1 for outermost


@dataclass
class NestedPlan:
    decline: str
    spans: List[Span] = field(default_factory=list)
    private_start_page: np.ndarray = None     # [B]
    merge_indptr: np.ndarray = None           # [B+1]
    spans_of: List[List[int]] = field(default_factory=list)   # per request, outermost first


def _child_spans(indptr, indices, kv_len, P, params, parent: Span, parent_index: int):
    e = parent.start_page + parent.span_pages
    by_page = {}
    for b in parent.members:
        if int(indptr[b + 1] - indptr[b]) > e:
            by_page.setdefault(int(indices[indptr[b] + e]), []).append(b)
    out = []
    for mem in by_page.values():
        mem = sorted(mem)
        if len(mem) < max(2, params.min_members):
            continue
        npages = [int(indptr[b + 1] - indptr[b]) for b in mem]
        c = 0
        while all(e + c < n for n in npages):
            pid = int(indices[indptr[mem[0]] + e + c])
            if any(int(indices[indptr[b] + e + c]) != pid for b in mem):
                break
            c += 1
        c = min([c] + [int(kv_len[b]) // P - e for b in mem])
        if c < max(1, params.min_shared_pages):
            continue
        if any(e + c == n for n in npages):
            continue
        out.append(Span(members=mem, start_page=e, span_pages=c, depth=parent.depth + 1,
                        parent=parent_index))
    return sorted(out, key=lambda s: s.members[0])


def build_nested_plan(indptr, indices, kv_len, page_size, params: planner.CascadeParams,
                      max_depth: int) -> NestedPlan:
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    B, P = len(kv_len), int(page_size)
    top = planner.build_cascade_plan(indptr, indices, kv_len, P, params)
    plan = NestedPlan(decline=top.decline)
    level = [Span(members=list(g.members), start_page=0, span_pages=g.span_pages, depth=0,
                  parent=-1) for g in top.groups]
    spans: List[Span] = []
    depth = 1
    while level:
        first = len(spans)
        spans += level
        if depth >= max_depth:
            break
        nxt = []
        for i, sp in enumerate(level):
            nxt += _child_spans(indptr, indices, kv_len, P, params, sp, first + i)
        level = sorted(nxt, key=lambda s: s.members[0])
        depth += 1
    plan.spans = spans
    spans_of = [[] for _ in range(B)]
    for i, sp in enumerate(spans):
        for b in sp.members:
            spans_of[b].append(i)
    for b in range(B):
        spans_of[b].sort(key=lambda i: spans[i].depth)
    plan.spans_of = spans_of
    start = np.zeros(B, dtype=np.int64)
    for b in range(B):
        if spans_of[b]:
            d = spans[spans_of[b][-1]]
            start[b] = d.start_page + d.span_pages
    plan.private_start_page = start.astype(np.int32)
    merge = [0]
    for b in range(B):
        merge.append(merge[-1] + len(spans_of[b]) + 1)
    plan.merge_indptr = np.asarray(merge, dtype=np.int32)
    return plan


def nested_cascade_decode(batch, params: planner.CascadeParams, max_depth: int,
                          return_plan=False):
    """Every request's states over its spans and its private range, merged
    (out [B, Hq, Dv], lse [B, Hq]). A span's state for a member is attention
    over the member's own tokens of that span, which are the span's shared
    pages."""
    plan = build_nested_plan(batch.indptr, batch.indices, batch.kv_len, batch.page_size, params,
                             max_depth)
    B, Hq, Dv, P = len(batch.kv_len), batch.num_q_heads, batch.head_dim_v, batch.page_size
    G = Hq // batch.num_kv_heads
    qf = decode(batch.q, batch.q_dtype)
    rows_v = np.zeros((int(plan.merge_indptr[-1]), Hq, Dv))
    rows_l = np.full((int(plan.merge_indptr[-1]), Hq), -np.inf)

    def state(b, a, e):
        K, V = attention.gather(batch.k_pool, batch.v_pool, batch.kv_dtype, batch.k_scale,
                                batch.v_scale, batch.indptr, batch.indices, batch.kv_len, P, b,
                                Dv, start=a, end=e)
        return attention.attend(qf[b], K, V, batch.sm_scale, G)

    for b in range(B):
        r = int(plan.merge_indptr[b])
        for i in plan.spans_of[b]:
            sp = plan.spans[i]
            rows_v[r], rows_l[r] = state(b, sp.start_page * P, (sp.start_page + sp.span_pages) * P)
            r += 1
        rows_v[r], rows_l[r] = state(b, int(plan.private_start_page[b]) * P, int(batch.kv_len[b]))
    out, lse = attention.merge_states(rows_v, rows_l, plan.merge_indptr)
    return (out, lse, plan) if return_plan else (out, lse)
