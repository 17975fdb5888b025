"""Plans the library must produce, written out from oracle/ (the planner
and the nested planner) for the plan tests: every field a plan exposes,
plus the library's single-merge row layout written from its reading."""
import numpy as np

from oracle import planner as oplan


def fused_rows(group_of, l0_len, l1_len, params):
    """The library's single-merge row layout, written out from its reading
    (not a rule of the page, which pairs one level-0 and one level-1 state
    per member): request b owns ceil(l0_len/S0) rows for the span holding it
    (none for a non-member), then max(1, ceil(l1_len/S1)) level-1 rows, so an
    empty level-1 range still owns the (0, -inf) row its merge reads."""
    S0, S1 = int(params.l0_partition_tokens), int(params.l1_partition_tokens)
    out = [0]
    for b in range(len(l1_len)):
        k = int(group_of[b])
        n0 = -(-int(l0_len[k]) // S0) if k >= 0 else 0
        out.append(out[-1] + n0 + max(1, -(-int(l1_len[b]) // S1)))
    return np.asarray(out, dtype=np.int32)


def nested_expected(indptr, indices, kv_len, P, params, depth):
    """The arrays the library's plan must hold, from the oracle's nested plan."""
    from oracle import nested
    ref = nested.build_nested_plan(indptr, indices, kv_len, P, params, depth)
    B = len(kv_len)
    members, gptr, l0_idx, l0_ptr = [], [0], [], [0]
    for sp in ref.spans:
        members += sp.members
        gptr.append(len(members))
        b0 = sp.members[0]
        l0_idx += list(indices[indptr[b0] + sp.start_page:indptr[b0] + sp.start_page + sp.span_pages])
        l0_ptr.append(len(l0_idx))
    group_of, rank = [-1] * B, [-1] * B
    for k, sp in enumerate(ref.spans):
        if sp.depth == 0:
            for m, b in enumerate(sp.members):
                group_of[b], rank[b] = k, m
    l1_idx, l1_ptr, l1_len = [], [0], []
    for b in range(B):
        s = int(ref.private_start_page[b])
        l1_idx += list(indices[indptr[b] + s:indptr[b + 1]])
        l1_ptr.append(len(l1_idx))
        l1_len.append(int(kv_len[b]) - s * P)
    return ref, {"members": members, "group_indptr": gptr,
                 "span_pages": [s.span_pages for s in ref.spans],
                 "span_start": [s.start_page for s in ref.spans],
                 "span_parent": [s.parent for s in ref.spans],
                 "l0_indptr": l0_ptr, "l0_indices": l0_idx,
                 "l0_len": [s.span_pages * P for s in ref.spans],
                 "l1_indptr": l1_ptr, "l1_indices": l1_idx, "l1_len": l1_len,
                 "merge_indptr": ref.merge_indptr, "group_of": group_of, "member_rank": rank}


ORACLE_KEYS = ("enabled", "min_shared_pages", "min_members", "max_groups",
               "l0_partition_tokens", "l1_partition_tokens")


def oracle_params(kw):
    return oplan.CascadeParams(**{k: v for k, v in kw.items() if k in ORACLE_KEYS})


def expected_plan(indptr, indices, kv_len, P, kw):
    """(fields, stats, decline) the library's plan must hold for the
    parameters kw (pdk.CascadeParams keywords), from oracle/planner.py for
    one span level and oracle/nested.py for max_depth > 1. stats is None for
    nested plans (checked field by field instead)."""
    op = oracle_params(kw)
    depth = int(kw.get("max_depth", 1))
    if depth > 1:
        ref, want = nested_expected(indptr, indices, kv_len, P, op, depth)
        rows = [0]
        S0, S1 = op.l0_partition_tokens, op.l1_partition_tokens
        for b, n1 in enumerate(want["l1_len"]):
            n0 = sum(-(-ref.spans[k].span_pages * P // S0) for k in ref.spans_of[b])
            rows.append(rows[-1] + n0 + max(1, -(-int(n1) // S1)))
        want["fused_merge_indptr"] = rows
        return want, None, ref.decline
    ref = oplan.build_cascade_plan(indptr, indices, kv_len, P, op)
    K = len(ref.span_pages)
    want = {f: getattr(ref, f) for f in ("members", "group_indptr", "span_pages", "l0_indptr",
                                         "l0_indices", "l0_len", "l1_indptr", "l1_indices",
                                         "l1_len", "merge_indptr", "group_of", "member_rank")}
    want["span_start"] = [0] * K
    want["span_parent"] = [-1] * K
    want["fused_merge_indptr"] = fused_rows(ref.group_of, ref.l0_len, ref.l1_len, op)
    return want, ref.stats, ref.decline
