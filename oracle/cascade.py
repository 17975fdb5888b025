"""Cascade (shared-prefix) decode composed from the definitions.

Test infrastructure only. Follows [cascade-PR] sections "The decomposition,
and the one part that is not obvious" and "Task items" (item 2): level 0
attends each selected group's shared span once, as one request whose query
heads are the members' heads stacked KV-head-major; level 1 attends every
request's remaining range; each member then merges its two states, and a
non-member's single state passes through a merge group of one.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from . import attention, planner
from .codecs import decode


def _view(batch, **over):
    fields = dict(k_pool=batch.k_pool, v_pool=batch.v_pool, kv_dtype=batch.kv_dtype,
                  k_scale=batch.k_scale, v_scale=batch.v_scale, page_size=batch.page_size,
                  num_q_heads=batch.num_q_heads, num_kv_heads=batch.num_kv_heads,
                  head_dim_k=batch.head_dim_k, head_dim_v=batch.head_dim_v,
                  q=batch.q, q_dtype=batch.q_dtype, sm_scale=batch.sm_scale,
                  partition_tokens=batch.partition_tokens, indptr=batch.indptr,
                  indices=batch.indices, kv_len=batch.kv_len)
    fields.update(over)
    return SimpleNamespace(**fields)


def level_state(batch, csr, partition_tokens, q=None, num_q_heads=None):
    """Per-request state of a level: partials over its view, then merged."""
    view = _view(batch, num_q_heads=num_q_heads or batch.num_q_heads)
    v, l, pind = attention.partial_attention(view, partition_tokens, csr=csr, q=q)
    return attention.merge_states(v, l, pind)


def cascade_decode(batch, params: planner.CascadeParams, head_map_fn=None, return_plan=False):
    """Cascade decode of ``batch`` (out [B, Hq, Dv], lse [B, Hq]).

    ``head_map_fn(M, Hkv, G)`` chooses the stacking (KV-head-major by default;
    the member-major map is the negative control)."""
    head_map_fn = head_map_fn or planner.stacked_head_map
    plan = planner.build_cascade_plan(batch.indptr, batch.indices, batch.kv_len,
                                      batch.page_size, params)
    B, Hq, Dv = len(batch.kv_len), batch.num_q_heads, batch.head_dim_v
    Hkv = batch.num_kv_heads
    G = Hq // Hkv
    qf = decode(batch.q, batch.q_dtype)

    # level 1 (the whole batch when the plan declined)
    out1, lse1 = level_state(batch, (plan.l1_indptr, plan.l1_indices, plan.l1_len),
                             params.l1_partition_tokens)
    if not plan.groups:
        return (out1, lse1, plan) if return_plan else (out1, lse1)

    # level 0: one stacked request per selected group
    out0 = {}
    for k, g in enumerate(plan.groups):
        M = len(g.members)
        hmap = head_map_fn(M, Hkv, G)               # h0 -> m*Hq + i
        q0 = np.empty((1, M * Hq, qf.shape[2]))
        for h0 in range(M * Hq):
            m, i = divmod(int(hmap[h0]), Hq)
            q0[0, h0] = qf[g.members[m], i]
        csr0 = (np.array([0, g.span_pages], np.int32),
                plan.l0_indices[plan.l0_indptr[k]:plan.l0_indptr[k + 1]],
                np.array([g.span_pages * batch.page_size], np.int32))
        o, l = level_state(batch, csr0, params.l0_partition_tokens, q=q0, num_q_heads=M * Hq)
        for h0 in range(M * Hq):
            m, i = divmod(int(hmap[h0]), Hq)
            out0[(g.members[m], i)] = (o[0, h0], l[0, h0])

    # pair merge: [level-0 state, level-1 state] for members, one row otherwise
    rows_v = np.zeros((int(plan.merge_indptr[-1]), Hq, Dv))
    rows_l = np.full((int(plan.merge_indptr[-1]), Hq), -np.inf)
    for b in range(B):
        r = int(plan.merge_indptr[b])
        if plan.group_of[b] >= 0:
            for i in range(Hq):
                rows_v[r, i], rows_l[r, i] = out0[(b, i)]
            r += 1
        rows_v[r], rows_l[r] = out1[b], lse1[b]
    out, lse = attention.merge_states(rows_v, rows_l, plan.merge_indptr)
    return (out, lse, plan) if return_plan else (out, lse)
