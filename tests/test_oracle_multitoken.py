"""Pins for the oracle's multi-token query steps (no GPU).

What pins what:
  * torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine) with an explicit boolean mask that lets query token t see
    positions <= n - T + t, on keys/values scattered into a paged pool by the
    test; and, where T equals the range length, the library's own
    ``is_causal`` mask (the square case, where its top-left alignment and
    the end alignment agree);
  * the single-token definition, already pinned: causal query token t equals
    one-token decode over the range truncated to n - T + t + 1 tokens, and
    T = 1 reduces to one-token decode;
  * brute force with math.fsum on tiny inputs;
  * the merge invariants [cascade-PR, "How the #898 merge kernel is reused"]:
    per-token partials merged equal the full multi-token result, with
    partitions that some query tokens see only in part or not at all;
  * the chunked split of [DCP-PR, section 3.2 figure] with T query tokens
    equals one causal softmax over prefix ++ suffix;
  * negative control: aligning the causal mask at the start of the range
    (query t sees positions <= t) misses the end-aligned result.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import attention, multitoken
from oracle.codecs import decode
from workloads import mla_decode_share, mla_share_with_query_tokens, random_batch, \
    with_query_tokens

LN2 = math.log(2.0)


def dense_mt_batch(rng, lens, T, Hq, Hkv, D, P, Dv=None, scale=None, pad=3):
    """Per-request keys/values scattered into a paged f32 pool through a
    random page table by this test, and T query tokens per request."""
    Dv = D if Dv is None else Dv
    Ks = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    Vs = [rng.standard_normal((n, Hkv, Dv)).astype(np.float32) for n in lens]
    npages = [-(-n // P) for n in lens]
    rows = rng.permutation(sum(npages) + pad)
    kpool = np.full((len(rows), Hkv, P, D), np.nan, np.float32)
    vpool = np.full((len(rows), Hkv, P, Dv), np.nan, np.float32)
    indptr, indices, r = [0], [], 0
    for b, n in enumerate(lens):
        ids = [int(x) for x in rows[r:r + npages[b]]]
        r += npages[b]
        indices += ids
        indptr.append(len(indices))
        for t in range(n):
            kpool[ids[t // P], :, t % P] = Ks[b][t]
            vpool[ids[t // P], :, t % P] = Vs[b][t]
    q = rng.standard_normal((len(lens), T, Hq, D)).astype(np.float32)
    batch = SimpleNamespace(k_pool=kpool, v_pool=vpool, kv_dtype="f32", k_scale=1.0,
                            v_scale=1.0, page_size=P, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_k=D, head_dim_v=Dv, q=q, q_dtype="f32",
                            sm_scale=(1 / math.sqrt(D)) if scale is None else scale,
                            partition_tokens=2 * P, indptr=np.array(indptr, np.int32),
                            indices=np.array(indices, np.int32),
                            kv_len=np.array(lens, np.int32))
    return batch, Ks, Vs


def sdpa_masked(batch, Ks, Vs, b, causal, library_causal=False):
    """Library attention for request b: [T, Hq, Dv] and log2 LSE [T, Hq]."""
    G = batch.num_q_heads // batch.num_kv_heads
    T, n = batch.q.shape[1], len(Ks[b])
    q = torch.from_numpy(batch.q[b].astype(np.float64)).permute(1, 0, 2)[None]      # [1,Hq,T,D]
    k = torch.from_numpy(Ks[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    v = torch.from_numpy(Vs[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    s = (q @ k.transpose(-1, -2)) * batch.sm_scale
    if library_causal:
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=batch.sm_scale,
                                                             is_causal=True)
        mask = torch.ones(T, n, dtype=torch.bool).tril()
    else:
        pos = torch.arange(n)[None, :]
        lim = (n - T + torch.arange(T))[:, None] if causal else torch.full((T, 1), n - 1)
        mask = pos <= lim
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                             scale=batch.sm_scale)
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1) / LN2
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [2, 4])
def test_multi_token_matches_torch_sdpa_with_mask(causal, T):
    rng = np.random.default_rng(300 + T + 10 * causal)
    lens = [T, 7, 16, 33]
    batch, Ks, Vs = dense_mt_batch(rng, lens, T, 8, 2, 16, 8)
    out, lse = multitoken.multi_token_attention(batch, causal)
    for b in range(len(lens)):
        ro, rl = sdpa_masked(batch, Ks, Vs, b, causal)
        assert np.max(np.abs(out[b] - ro)) < 1e-12
        assert np.max(np.abs(lse[b] - rl)) < 1e-12


def test_square_case_matches_the_library_causal_mask():
    rng = np.random.default_rng(310)
    lens = [5, 5]
    batch, Ks, Vs = dense_mt_batch(rng, lens, 5, 4, 2, 8, 4)
    out, lse = multitoken.multi_token_attention(batch, True)
    for b in range(2):
        ro, rl = sdpa_masked(batch, Ks, Vs, b, True, library_causal=True)
        assert np.max(np.abs(out[b] - ro)) < 1e-12
        assert np.max(np.abs(lse[b] - rl)) < 1e-12


def test_causal_token_equals_truncated_single_token_decode():
    b = with_query_tokens(random_batch(320, batch=5, page_size=16, num_q_heads=8, num_kv_heads=2,
                                       head_dim=32, kv_dtype="bf16", q_dtype="bf16",
                                       min_len=3, max_len=90, partition_tokens=32), 3, 321)
    out, lse = multitoken.multi_token_attention(b, True)
    qf = decode(b.q, b.q_dtype)
    for t in range(3):
        kv_t = np.maximum(b.kv_len - 3 + t + 1, 0).astype(np.int32)
        so, sl = attention.decode_attention(b, csr=(b.indptr, b.indices, kv_t), q=qf[:, t])
        assert np.array_equal(out[:, t], so) and np.array_equal(lse[:, t], sl)


def test_one_token_step_is_single_token_decode():
    base = random_batch(330, batch=4, page_size=8, num_q_heads=4, num_kv_heads=1, head_dim=16,
                        kv_dtype="f32", q_dtype="f32", min_len=1, max_len=40,
                        partition_tokens=16)
    b = with_query_tokens(base, 1, 331)
    so, sl = attention.decode_attention(b, q=decode(b.q, b.q_dtype)[:, 0])
    for causal in (True, False):
        out, lse = multitoken.multi_token_attention(b, causal)
        assert np.array_equal(out[:, 0], so) and np.array_equal(lse[:, 0], sl)


def test_brute_force_tiny():
    rng = np.random.default_rng(340)
    for trial in range(12):
        T = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 7, size=2)]
        batch, Ks, Vs = dense_mt_batch(rng, lens, T, 2, 1, 3, 2, Dv=2)
        out, lse = multitoken.multi_token_attention(batch, True)
        for b, n in enumerate(lens):
            for t in range(T):
                seen = n - T + t + 1
                for i in range(2):
                    if seen <= 0:
                        assert np.all(out[b, t, i] == 0) and lse[b, t, i] == -np.inf
                        continue
                    s = [batch.sm_scale * math.fsum(float(batch.q[b, t, i, d]) *
                                                    float(Ks[b][p, 0, d]) for d in range(3))
                         for p in range(seen)]
                    m = max(s)
                    e = [math.exp(x - m) for x in s]
                    l = math.fsum(e)
                    for d in range(2):
                        want = math.fsum(e[p] * float(Vs[b][p, 0, d]) for p in range(seen)) / l
                        assert abs(out[b, t, i, d] - want) < 1e-13
                    assert abs(lse[b, t, i] - (m + math.log(l)) / LN2) < 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_token_partials_merge_to_the_full_result(causal):
    # partitions of 8 tokens, 4 query tokens: the last partition of a short
    # request is invisible to the early query tokens (empty states)
    base = random_batch(350, batch=6, page_size=4, num_q_heads=4, num_kv_heads=2, head_dim=16,
                        kv_dtype="bf16", q_dtype="bf16", min_len=1, max_len=45,
                        partition_tokens=8, lens=[1, 3, 9, 17, 24, 45])
    b = with_query_tokens(base, 4, 351)
    v, l, pind = multitoken.multi_token_partials(b, causal, 8)
    if causal:
        assert np.any(l == -np.inf)
    mo, ml = multitoken.merge_token_states(v, l, pind)
    fo, fl = multitoken.multi_token_attention(b, causal)
    assert np.max(np.abs(mo - fo)) < 1e-12
    empty = fl == -np.inf     # query tokens that see nothing (a 1-token request)
    assert np.array_equal(ml == -np.inf, empty) and np.all(mo[empty] == 0)
    assert np.max(np.abs(ml[~empty] - fl[~empty])) < 1e-12


def test_mla_multi_token_composition_equals_flat():
    share = mla_share_with_query_tokens(
        mla_decode_share(batch=2, heads=4, context=512, suffix_tokens=64, chunk_tokens=128,
                         page_size=64, partition_tokens=64, suffix_partition_tokens=32), 3, 360)
    out, lse = multitoken.mla_multi_token(share)
    fo, fl = multitoken.mla_multi_token_flat(share)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12
    assert np.all(np.isfinite(out))


def test_start_aligned_causal_mask_misses():
    rng = np.random.default_rng(370)
    lens = [12, 20]
    batch, Ks, Vs = dense_mt_batch(rng, lens, 3, 4, 2, 8, 4)
    out, _ = multitoken.multi_token_attention(batch, True)
    for b, n in enumerate(lens):
        G = 2
        for t in range(3):
            seen = t + 1          # the wrong reading: query t sees positions <= t
            for i in range(4):
                K = Ks[b][:seen, i // G].astype(np.float64)
                V = Vs[b][:seen, i // G].astype(np.float64)
                s = batch.sm_scale * (K @ batch.q[b, t, i].astype(np.float64))
                w = np.exp(s - s.max())
                wrong = (w @ V) / w.sum()
                assert np.max(np.abs(out[b, t, i] - wrong)) > 1e-3
