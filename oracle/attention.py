"""Paged decode attention, partials and the log2-LSE merge, by definition.

Test infrastructure only (see the package docstring). Everything is float64,
computed from the exact stored values (after the fp8 -> bf16 dequant where the
pool is fp8).

Definitions followed:
  * One query token per request. Query head ``i`` reads KV head ``i // G``
    with ``G = Hq / Hkv`` [cascade-PR, "The decomposition, and the one part
    that is not obvious": query head h maps to KV head h / NRep].
  * Token ``t`` of request ``b`` is slot ``t % P`` of pool row
    ``indices[indptr[b] + t // P]``; only tokens ``t < kv_len[b]`` exist.
  * A state over a key range is the softmax-weighted mean of the values,
    normalized by its own denominator, plus its log-sum-exp in log2 units,
    ``log2 sum_t 2^(s_t * log2 e)`` = ``m + log2 l`` in the page's notation
    [cascade-PR, "How the #898 merge kernel is reused": partials arrive
    normalized, the LSE is m + log2(l)]. An empty range is the state
    (out = 0, lse = -inf).
  * Partitions tile each request's range from its first token in
    ``partition_tokens`` steps; the last one may be short (reading: the pages
    leave the boundaries to the heuristic chunk size).
  * Merging rows ``r`` of a group: m = max lse_r, w_r = 2^(lse_r - m),
    l = sum w_r, out = sum w_r v_r / l, lse = m + log2 l. Rows with
    lse = -inf take no part; a group with none left is (0, -inf). A group of
    one row gives w = 1, l = 1, out = v: the identity the page relies on to
    let non-members ride along [cascade-PR, "How the #898 merge kernel is
    reused"].
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import decode

LOG2E = 1.0 / math.log(2.0)


# --------------------------------------------------------------------------
# Gathering a request's keys and values through the page table
# --------------------------------------------------------------------------

def gather(k_pool, v_pool, kv_dtype, k_scale, v_scale, indptr, indices, kv_len,
           page_size, b, head_dim_v, start=0, end=None):
    """K [n, Hkv, Dk] and V [n, Hkv, Dv] (float64) of request ``b`` for tokens
    ``start <= t < end`` (``end`` defaults to ``kv_len[b]``).

    ``k_pool``/``v_pool`` are HND raw storage ``[rows, Hkv, P, D]``; with
    ``v_pool is None`` the values are the first ``head_dim_v`` lanes of K
    (one latent row serves as key and value)."""
    n = int(kv_len[b])
    end = n if end is None else min(int(end), n)
    start = int(start)
    if end <= start:
        hk = k_pool.shape[1]
        return (np.zeros((0, hk, k_pool.shape[3])), np.zeros((0, hk, head_dim_v)))
    ids = np.asarray(indices[int(indptr[b]):int(indptr[b + 1])])
    t = np.arange(start, end)
    rows = ids[t // page_size]
    slots = t % page_size
    K = decode(k_pool[rows, :, slots, :], kv_dtype, k_scale)     # [n, Hkv, Dk]
    if v_pool is None:
        V = K[:, :, :head_dim_v]
    else:
        V = decode(v_pool[rows, :, slots, :], kv_dtype, v_scale)
    return K, V


def attend(q_heads, K, V, scale, group):
    """Softmax attention of ``q_heads`` [Hq, Dk] over keys K [n, Hkv, Dk] and
    values V [n, Hkv, Dv]. Returns out [Hq, Dv] and lse in log2 units [Hq]."""
    Hq = q_heads.shape[0]
    Dv = V.shape[2]
    out = np.zeros((Hq, Dv))
    lse = np.full(Hq, -np.inf)
    if K.shape[0] == 0:
        return out, lse
    for i in range(Hq):
        kv = i // group
        s = scale * (K[:, kv, :] @ q_heads[i])     # natural-log scores
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[i] = (e @ V[:, kv, :]) / l
        lse[i] = (m + math.log(l)) * LOG2E
    return out, lse


def _q(batch):
    return decode(batch.q, batch.q_dtype)


def _csr(batch, csr):
    if csr is None:
        return batch.indptr, batch.indices, batch.kv_len
    return csr


def decode_attention(batch, csr=None, requests=None, q=None):
    """Flat attention over each request's whole range.

    ``batch`` supplies the pool, queries, heads, page size and scale; ``csr``
    (indptr, indices, kv_len) overrides its page table. ``requests`` limits
    the work to a subset. Returns out [B, Hq, Dv] and lse [B, Hq] (rows not
    computed are left NaN)."""
    indptr, indices, kv_len = _csr(batch, csr)
    qf = _q(batch) if q is None else q
    B = len(kv_len)
    Hq, Dv = batch.num_q_heads, batch.head_dim_v
    G = Hq // batch.num_kv_heads
    out = np.full((B, Hq, Dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        K, V = gather(batch.k_pool, batch.v_pool, batch.kv_dtype, batch.k_scale,
                      batch.v_scale, indptr, indices, kv_len, batch.page_size, b, Dv)
        out[b], lse[b] = attend(qf[b], K, V, batch.sm_scale, G)
    return out, lse


# --------------------------------------------------------------------------
# Partitions (split-KV) and partial states
# --------------------------------------------------------------------------

def partition_indptr(kv_len, partition_tokens):
    """part_indptr[b+1] = part_indptr[b] + ceil(kv_len[b] / partition_tokens)."""
    S = int(partition_tokens)
    out = np.zeros(len(kv_len) + 1, dtype=np.int64)
    for b, n in enumerate(kv_len):
        out[b + 1] = out[b] + (int(n) + S - 1) // S
    return out.astype(np.int32)


def partial_attention(batch, partition_tokens=None, csr=None, q=None):
    """One state per (request, partition): partition p of request b covers
    tokens [p*S, min((p+1)*S, kv_len[b])). Returns v_part [R, Hq, Dv],
    lse_part [R, Hq] and part_indptr [B+1]; row = part_indptr[b] + p."""
    indptr, indices, kv_len = _csr(batch, csr)
    S = int(batch.partition_tokens if partition_tokens is None else partition_tokens)
    qf = _q(batch) if q is None else q
    Hq, Dv = batch.num_q_heads, batch.head_dim_v
    G = Hq // batch.num_kv_heads
    pind = partition_indptr(kv_len, S)
    R = int(pind[-1])
    v_part = np.zeros((R, Hq, Dv))
    lse_part = np.full((R, Hq), -np.inf)
    for b in range(len(kv_len)):
        for p in range(int(pind[b + 1] - pind[b])):
            K, V = gather(batch.k_pool, batch.v_pool, batch.kv_dtype, batch.k_scale,
                          batch.v_scale, indptr, indices, kv_len, batch.page_size, b, Dv,
                          start=p * S, end=(p + 1) * S)
            r = int(pind[b]) + p
            v_part[r], lse_part[r] = attend(qf[b], K, V, batch.sm_scale, G)
    return v_part, lse_part, pind


# --------------------------------------------------------------------------
# Merge of states
# --------------------------------------------------------------------------

def merge_states(v_in, lse_in, o_indptr):
    """Merge contiguous row groups: output row j combines input rows
    o_indptr[j] <= r < o_indptr[j+1]. v_in [N, H, D], lse_in [N, H] in log2
    units; returns v_out [M, H, D] and lse_out [M, H] (float64)."""
    v_in = np.asarray(v_in, dtype=np.float64)
    lse_in = np.asarray(lse_in, dtype=np.float64)
    M = len(o_indptr) - 1
    H, D = v_in.shape[1], v_in.shape[2]
    v_out = np.zeros((M, H, D))
    lse_out = np.full((M, H), -np.inf)
    for j in range(M):
        a, e = int(o_indptr[j]), int(o_indptr[j + 1])
        for h in range(H):
            ls = lse_in[a:e, h]
            live = ls > -np.inf
            if not np.any(live):
                continue
            m = ls[live].max()
            w = np.exp2(ls[live] - m)
            l = w.sum()
            v_out[j, h] = (w @ v_in[a:e, h][live]) / l
            lse_out[j, h] = m + math.log2(l)
    return v_out, lse_out
