"""Multi-token query steps: T query tokens per request in one step.

Test infrastructure only (see the package docstring). Float64 throughout,
built on the single-token definitions of ``attention.py`` (gather, attend,
partitions, merge).

Definitions followed:
  * A step carries T >= 1 query tokens per request, ``q [B, T, Hq, Dk]``.
    The request's range (``kv_len`` tokens) already holds the step's T new
    tokens as its last T tokens, so query token t sits at position
    ``kv_len - T + t``.
  * Causal: query token t sees the tokens at positions ``0 .. kv_len - T + t``
    (itself and everything before it). This is the new-token self-attention
    whose state [DCP-PR, section 3.2 figure] merges with the cached-prefix
    state last; the page names only the cached chunks' call
    (``causal=False``), so the causal rule for the new tokens is the reading
    that makes the composition equal one causal softmax over the whole
    sequence.
  * Non-causal: every query token sees the whole range - the cached prefix
    chunks of [DCP-PR, section 3.2 figure], attended with ``causal=False``.
  * Readings: T is the same for every request of a step; a query token whose
    visible range is empty (``kv_len - T + t + 1 <= 0``) has the empty state
    (out = 0, lse = -inf); partitions tile the range exactly as for one token
    and each query token's partial covers the part of the partition it sees.
  * The T query tokens take the place of T x Hq heads in the merge: states are
    ``[R, T, Hq, Dv]`` / ``[R, T, Hq]`` and a merge over them is the
    single-token merge with ``H = T * Hq`` [cascade-PR, "How the #898 merge
    kernel is reused": the merge combines rows head by head].
"""
from __future__ import annotations

import numpy as np

from . import attention
from .codecs import decode


def visible_end(kv_len: int, q_tokens: int, t: int, causal: bool) -> int:
    """Exclusive end of the positions query token ``t`` sees."""
    n = int(kv_len)
    if not causal:
        return n
    return max(0, n - int(q_tokens) + int(t) + 1)


def _queries(batch, q):
    qf = decode(batch.q, batch.q_dtype) if q is None else np.asarray(q, np.float64)
    assert qf.ndim == 4, "multi-token queries are [B, T, Hq, Dk]"
    return qf


def multi_token_attention(batch, causal: bool, csr=None, q=None, requests=None):
    """Full attention of every query token of every request over the range it
    sees. Returns out [B, T, Hq, Dv] and lse [B, T, Hq] (rows not computed
    are NaN)."""
    indptr, indices, kv_len = attention._csr(batch, csr)
    qf = _queries(batch, q)
    B, T = qf.shape[0], qf.shape[1]
    Hq, Dv = batch.num_q_heads, batch.head_dim_v
    G = Hq // batch.num_kv_heads
    out = np.full((B, T, Hq, Dv), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        for t in range(T):
            end = visible_end(kv_len[b], T, t, causal)
            K, V = attention.gather(batch.k_pool, batch.v_pool, batch.kv_dtype, batch.k_scale,
                                    batch.v_scale, indptr, indices, kv_len, batch.page_size, b,
                                    Dv, start=0, end=end)
            out[b, t], lse[b, t] = attention.attend(qf[b, t], K, V, batch.sm_scale, G)
    return out, lse


def multi_token_partials(batch, causal: bool, partition_tokens=None, csr=None, q=None):
    """One state per (request, partition, query token): partition p of
    request b covers positions [p*S, min((p+1)*S, kv_len[b])) and query
    token t keeps the part of it below its visible end. Returns v_part
    [R, T, Hq, Dv], lse_part [R, T, Hq] and part_indptr [B+1]."""
    indptr, indices, kv_len = attention._csr(batch, csr)
    S = int(batch.partition_tokens if partition_tokens is None else partition_tokens)
    qf = _queries(batch, q)
    T = qf.shape[1]
    Hq, Dv = batch.num_q_heads, batch.head_dim_v
    G = Hq // batch.num_kv_heads
    pind = attention.partition_indptr(kv_len, S)
    R = int(pind[-1])
    v_part = np.zeros((R, T, Hq, Dv))
    lse_part = np.full((R, T, Hq), -np.inf)
    for b in range(len(kv_len)):
        for p in range(int(pind[b + 1] - pind[b])):
            r = int(pind[b]) + p
            for t in range(T):
                end = min((p + 1) * S, visible_end(kv_len[b], T, t, causal))
                K, V = attention.gather(batch.k_pool, batch.v_pool, batch.kv_dtype,
                                        batch.k_scale, batch.v_scale, indptr, indices, kv_len,
                                        batch.page_size, b, Dv, start=p * S, end=end)
                v_part[r, t], lse_part[r, t] = attention.attend(qf[b, t], K, V, batch.sm_scale, G)
    return v_part, lse_part, pind


def merge_token_states(v_in, lse_in, o_indptr):
    """The log2-LSE merge of [N, T, Hq, Dv] states, each (token, head) pair a
    head of the single-token merge. Returns [M, T, Hq, Dv] and [M, T, Hq]."""
    v_in = np.asarray(v_in, np.float64)
    N, T, Hq, Dv = v_in.shape
    vo, lo = attention.merge_states(v_in.reshape(N, T * Hq, Dv),
                                    np.asarray(lse_in, np.float64).reshape(N, T * Hq), o_indptr)
    M = vo.shape[0]
    return vo.reshape(M, T, Hq, Dv), lo.reshape(M, T, Hq)


def mla_multi_token(share, q=None):
    """The chunked cached-prefix / new-suffix split of [DCP-PR, section 3.2
    figure] with T query tokens: every cached chunk non-causally (a chunk's
    state is the merge of its partitions), the chunk states merged, the
    new-token suffix causally, then the pair merge. Returns out
    [B, T, Hq, Dv] and lse [B, T, Hq]."""
    from . import mla
    pre, suf = share.prefix, share.suffix
    qf = _queries(pre, q)
    csr, cptr = mla.chunk_csr(pre, share.chunk_tokens)
    q_chunks = np.repeat(qf, np.diff(cptr), axis=0)
    v, l, pind = multi_token_partials(pre, False, pre.partition_tokens, csr=csr, q=q_chunks)
    chunk_out, chunk_lse = merge_token_states(v, l, pind)
    pre_out, pre_lse = merge_token_states(chunk_out, chunk_lse, cptr)
    sv, sl, spind = multi_token_partials(suf, True, suf.partition_tokens, q=qf)
    suf_out, suf_lse = merge_token_states(sv, sl, spind)
    B = qf.shape[0]
    rows_v = np.stack([pre_out, suf_out], axis=1).reshape(2 * B, *pre_out.shape[1:])
    rows_l = np.stack([pre_lse, suf_lse], axis=1).reshape(2 * B, *pre_lse.shape[1:])
    return merge_token_states(rows_v, rows_l, np.arange(0, 2 * B + 1, 2))


def mla_multi_token_flat(share, q=None, requests=None):
    """The plain definition: for query token t one softmax over the whole
    cached prefix followed by the suffix positions it sees causally."""
    pre, suf = share.prefix, share.suffix
    qf = _queries(pre, q)
    B, T = qf.shape[0], qf.shape[1]
    Hq, Dv = pre.num_q_heads, pre.head_dim_v
    out = np.full((B, T, Hq, Dv), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        K1, V1 = attention.gather(pre.k_pool, pre.v_pool, pre.kv_dtype, pre.k_scale, pre.v_scale,
                                  pre.indptr, pre.indices, pre.kv_len, pre.page_size, b, Dv)
        for t in range(T):
            end = visible_end(suf.kv_len[b], T, t, True)
            K2, V2 = attention.gather(suf.k_pool, suf.v_pool, suf.kv_dtype, suf.k_scale,
                                      suf.v_scale, suf.indptr, suf.indices, suf.kv_len,
                                      suf.page_size, b, Dv, start=0, end=end)
            out[b, t], lse[b, t] = attention.attend(qf[b, t], np.concatenate([K1, K2]),
                                                    np.concatenate([V1, V2]), pre.sm_scale,
                                                    Hq // pre.num_kv_heads)
    return out, lse
