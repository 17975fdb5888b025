"""Chunked cached-prefix / new-suffix decode of an MLA share.

Test infrastructure only. Follows [DCP-PR] section 3.2 (the cached-prefix
pipeline figure): the cached prefix is processed chunk by chunk, each chunk
returns an output and its LSE, the chunk states are LSE-merged, and that
result is LSE-merged with the state of the step's new (suffix) tokens. Here
all LSEs are in log2 units, so no unit conversion is applied anywhere
[cascade-PR, "How the #898 merge kernel is reused"]. The latent pool holds
one KV head whose first 512 lanes are the values; fp8 rows are dequantized
to bf16 with the per-tensor scale before use [DCP-PR, 3.3].

Reading: a chunk state is itself the merge of that chunk's partitions
(sub-partitions of ``prefix.partition_tokens`` tokens); chunks are aligned at
token 0 of the cached range.
"""
from __future__ import annotations

import numpy as np

from . import attention
from .codecs import decode


def chunk_csr(batch, chunk_tokens):
    """Each (request, chunk) as its own pseudo-request, request-major:
    chunk c of request b covers tokens [c*C, min((c+1)*C, len)). Returns the
    CSR of the pseudo-requests and chunk_indptr [B+1] over them."""
    P = batch.page_size
    C = int(chunk_tokens)
    assert C % P == 0
    indptr, idx, lens, cptr = [0], [], [], [0]
    for b in range(len(batch.kv_len)):
        n = int(batch.kv_len[b])
        ids = batch.indices[batch.indptr[b]:batch.indptr[b + 1]]
        nch = -(-n // C)
        for c in range(nch):
            a, e = c * C, min((c + 1) * C, n)
            idx += [int(x) for x in ids[a // P:-(-e // P)]]
            indptr.append(len(idx))
            lens.append(e - a)
        cptr.append(cptr[-1] + nch)
    return (np.asarray(indptr, np.int32), np.asarray(idx, np.int32),
            np.asarray(lens, np.int32)), np.asarray(cptr, np.int32)


def mla_decode(share):
    """Returns (out [B, Hq, Dv], lse [B, Hq], chunk_out, chunk_lse)."""
    pre, suf = share.prefix, share.suffix
    csr, cptr = chunk_csr(pre, share.chunk_tokens)
    qf = decode(pre.q, pre.q_dtype)
    q_chunks = np.repeat(qf, np.diff(cptr), axis=0)
    v, l, pind = attention.partial_attention(pre, pre.partition_tokens, csr=csr, q=q_chunks)
    chunk_out, chunk_lse = attention.merge_states(v, l, pind)        # one state per chunk
    pre_out, pre_lse = attention.merge_states(chunk_out, chunk_lse, cptr)   # across chunks
    sv, sl, spind = attention.partial_attention(suf, suf.partition_tokens)
    suf_out, suf_lse = attention.merge_states(sv, sl, spind)
    B = len(pre.kv_len)
    rows_v = np.stack([pre_out, suf_out], axis=1).reshape(2 * B, *pre_out.shape[1:])
    rows_l = np.stack([pre_lse, suf_lse], axis=1).reshape(2 * B, -1)
    out, lse = attention.merge_states(rows_v, rows_l, np.arange(0, 2 * B + 1, 2))
    return out, lse, chunk_out, chunk_lse


def mla_flat(share, requests=None):
    """The plain definition: one softmax over prefix and suffix tokens together."""
    pre, suf = share.prefix, share.suffix
    qf = decode(pre.q, pre.q_dtype)
    B, Hq, Dv = len(pre.kv_len), pre.num_q_heads, pre.head_dim_v
    out = np.full((B, Hq, Dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        K1, V1 = attention.gather(pre.k_pool, pre.v_pool, pre.kv_dtype, pre.k_scale, pre.v_scale,
                                  pre.indptr, pre.indices, pre.kv_len, pre.page_size, b, Dv)
        K2, V2 = attention.gather(suf.k_pool, suf.v_pool, suf.kv_dtype, suf.k_scale, suf.v_scale,
                                  suf.indptr, suf.indices, suf.kv_len, suf.page_size, b, Dv)
        out[b], lse[b] = attention.attend(qf[b], np.concatenate([K1, K2]),
                                          np.concatenate([V1, V2]), pre.sm_scale,
                                          Hq // pre.num_kv_heads)
    return out, lse
