"""Pins for the oracle's attention, partials and merge (no GPU).

What pins what:
  * full attention vs torch's scaled_dot_product_attention in float64 on the
    CPU (a library routine), on keys/values scattered into a paged pool by
    this test and gathered back by the oracle;
  * closed forms: one key, zero scale, identical keys;
  * brute force with math.fsum on tiny inputs;
  * the invariants of the cascade page [cascade-PR, "The decomposition" and
    "How the #898 merge kernel is reused"]: merged disjoint-range partials
    equal flat attention, a one-row group is the identity, the merge is
    associative across regroupings, and natural-log LSEs fed to the log2
    merge give a wrong answer (negative control).
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import attention
from workloads import random_batch, tiny_gqa_fp32

LN2 = math.log(2.0)


def dense_batch(rng, lens, Hq, Hkv, D, P, Dv=None, scale=None, pad=3):
    """Keys/values drawn per request, then scattered into a paged f32 pool
    through a random page table (written independently of the oracle)."""
    Dv = D if Dv is None else Dv
    Ks = [rng.standard_normal((n, Hkv, D)) .astype(np.float32) for n in lens]
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
            pg, sl = ids[t // P], t % P
            for h in range(Hkv):
                kpool[pg, h, sl] = Ks[b][t, h]
                vpool[pg, h, sl] = Vs[b][t, h]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    batch = SimpleNamespace(k_pool=kpool, v_pool=vpool, kv_dtype="f32", k_scale=1.0,
                            v_scale=1.0, page_size=P, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_k=D, head_dim_v=Dv, q=q, q_dtype="f32",
                            sm_scale=(1 / math.sqrt(D)) if scale is None else scale,
                            partition_tokens=2 * P, indptr=np.array(indptr, np.int32),
                            indices=np.array(indices, np.int32),
                            kv_len=np.array(lens, np.int32))
    return batch, Ks, Vs


def sdpa_reference(batch, Ks, Vs):
    G = batch.num_q_heads // batch.num_kv_heads
    outs, lses = [], []
    for b in range(len(Ks)):
        q = torch.from_numpy(batch.q[b].astype(np.float64))[None, :, None, :]
        k = torch.from_numpy(Ks[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        v = torch.from_numpy(Vs[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=batch.sm_scale)
        s = (q @ k.transpose(-1, -2)) * batch.sm_scale
        outs.append(o[0, :, 0].numpy())
        lses.append((torch.logsumexp(s, dim=-1)[0, :, 0] / LN2).numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (6, 1)])
def test_flat_attention_matches_torch_sdpa(Hq, Hkv):
    rng = np.random.default_rng(11 + Hq)
    batch, Ks, Vs = dense_batch(rng, [1, 7, 16, 33, 50], Hq, Hkv, 16, 8)
    out, lse = attention.decode_attention(batch)
    ro, rl = sdpa_reference(batch, Ks, Vs)
    assert np.max(np.abs(out - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_one_key_closed_form():
    rng = np.random.default_rng(3)
    batch, Ks, Vs = dense_batch(rng, [1, 1], 4, 2, 8, 4)
    out, lse = attention.decode_attention(batch)
    for b in range(2):
        for i in range(4):
            kv = i // 2
            s = batch.sm_scale * float(np.dot(batch.q[b, i].astype(np.float64), Ks[b][0, kv]))
            assert np.array_equal(out[b, i], Vs[b][0, kv].astype(np.float64))
            assert abs(lse[b, i] - s / LN2) < 1e-14


def test_zero_scale_is_the_mean_and_log2_length():
    rng = np.random.default_rng(4)
    batch, Ks, Vs = dense_batch(rng, [5, 12], 4, 2, 8, 4, scale=0.0)
    out, lse = attention.decode_attention(batch)
    for b, n in enumerate([5, 12]):
        for i in range(4):
            assert np.allclose(out[b, i], Vs[b][:, i // 2].astype(np.float64).mean(0), atol=1e-14)
            assert abs(lse[b, i] - math.log2(n)) < 1e-13


def test_identical_keys_give_the_mean():
    rng = np.random.default_rng(5)
    batch, Ks, Vs = dense_batch(rng, [9], 2, 1, 8, 4)
    batch.k_pool[:] = batch.k_pool[batch.indices[0], 0, 0]
    out, _ = attention.decode_attention(batch)
    for i in range(2):
        assert np.allclose(out[0, i], Vs[0][:, 0].astype(np.float64).mean(0), atol=1e-14)


def test_brute_force_tiny():
    rng = np.random.default_rng(6)
    for trial in range(20):
        lens = [int(x) for x in rng.integers(1, 7, size=3)]
        batch, Ks, Vs = dense_batch(rng, lens, 4, 2, 3, 2, Dv=4)
        out, lse = attention.decode_attention(batch)
        for b, n in enumerate(lens):
            for i in range(4):
                kv = i // 2
                s = [batch.sm_scale * math.fsum(float(batch.q[b, i, d]) * float(Ks[b][t, kv, d])
                                                for d in range(3)) for t in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = math.fsum(e)
                for d in range(4):
                    want = math.fsum(e[t] * float(Vs[b][t, kv, d]) for t in range(n)) / l
                    assert abs(out[b, i, d] - want) < 1e-13
                assert abs(lse[b, i] - (m + math.log(l)) / LN2) < 1e-13


def test_partition_indptr_closed_form():
    lens = np.array([0, 1, 31, 32, 33, 64, 100])
    assert list(attention.partition_indptr(lens, 32)) == [0, 0, 1, 2, 3, 5, 7, 11]


def test_partials_merge_to_flat():
    b = random_batch(21, batch=5, page_size=8, num_q_heads=8, num_kv_heads=2, head_dim=16,
                     kv_dtype="bf16", q_dtype="bf16", min_len=1, max_len=90,
                     partition_tokens=16)
    flat_o, flat_l = attention.decode_attention(b)
    v, l, pind = attention.partial_attention(b)
    mo, ml = attention.merge_states(v, l, pind)
    assert np.max(np.abs(mo - flat_o)) < 1e-12
    assert np.max(np.abs(ml - flat_l)) < 1e-12
    assert np.all(np.isfinite(mo))  # poisoned slots were never read


def test_tiny_workload_partials_merge_to_flat():
    b = tiny_gqa_fp32()
    flat_o, flat_l = attention.decode_attention(b)
    v, l, pind = attention.partial_attention(b)
    assert list(pind) == [0, 2, 4, 7, 9]
    mo, ml = attention.merge_states(v, l, pind)
    assert np.max(np.abs(mo - flat_o)) < 1e-12 and np.max(np.abs(ml - flat_l)) < 1e-12


def test_merge_group_of_one_is_bit_exact_identity():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((5, 3, 8)).astype(np.float32)
    l = rng.uniform(-4, 20, (5, 3)).astype(np.float32)
    mo, ml = attention.merge_states(v, l, np.arange(6))
    assert np.array_equal(mo, v.astype(np.float64))
    assert np.array_equal(ml, l.astype(np.float64))


def test_merge_is_associative_across_regroupings():
    rng = np.random.default_rng(9)
    counts = rng.integers(1, 9, size=40)
    ind = np.concatenate([[0], np.cumsum(counts)])
    v = rng.standard_normal((ind[-1], 4, 8))
    l = rng.uniform(-4, 20, (ind[-1], 4))
    ref_o, ref_l = attention.merge_states(v, l, ind)
    for trial in range(5):
        # split every group into random contiguous subgroups, merge in two stages
        sub = [0]
        outer = [0]
        for j in range(len(counts)):
            a, e = ind[j], ind[j + 1]
            cuts = sorted(set(rng.integers(a + 1, e + 1, size=rng.integers(0, 3)).tolist()) | {e})
            sub += cuts
            outer.append(len(sub) - 1)
        so, sl = attention.merge_states(v, l, np.array(sub))
        o2, l2 = attention.merge_states(so, sl, np.array(outer))
        assert np.max(np.abs(o2 - ref_o)) < 1e-12
        assert np.max(np.abs(l2 - ref_l)) < 1e-12


def test_natural_log_lse_fails_the_log2_merge():
    """Negative control: natural-log LSEs through the log2 merge are wrong."""
    b = random_batch(22, batch=4, page_size=8, num_q_heads=4, num_kv_heads=1, head_dim=16,
                     kv_dtype="f32", q_dtype="f32", min_len=40, max_len=64,
                     partition_tokens=8)
    b.sm_scale = 1.0  # spread the partition LSEs well apart
    flat_o, _ = attention.decode_attention(b)
    v, l, pind = attention.partial_attention(b)
    good, _ = attention.merge_states(v, l, pind)
    bad, _ = attention.merge_states(v, l * LN2, pind)
    spread = max(np.ptp(l[pind[i]:pind[i + 1]], axis=0).max() for i in range(4))
    assert spread >= 4
    assert np.max(np.abs(good - flat_o)) < 1e-12
    assert np.max(np.abs(bad - flat_o)) > 100 * 1e-5


def test_merge_skips_empty_and_minus_inf_rows():
    v = np.array([[[1.0, 2.0]], [[np.nan, np.nan]], [[3.0, 4.0]]])
    l = np.array([[2.0], [-np.inf], [2.0]])
    mo, ml = attention.merge_states(v, l, np.array([0, 3, 3, 4]))
    assert np.allclose(mo[0, 0], [2.0, 3.0]) and ml[0, 0] == 3.0
    assert np.array_equal(mo[1], np.zeros((1, 2))) and ml[1, 0] == -np.inf   # empty group
    assert np.array_equal(mo[2], np.zeros((1, 2))) and ml[2, 0] == -np.inf   # only -inf


def test_empty_request_state():
    b = random_batch(23, batch=3, page_size=8, num_q_heads=2, num_kv_heads=1, head_dim=8,
                     kv_dtype="f32", q_dtype="f32", min_len=0, max_len=0,
                     partition_tokens=8, lens=[0, 5, 0])
    out, lse = attention.decode_attention(b)
    assert np.array_equal(out[0], np.zeros((2, 8))) and np.all(lse[0] == -np.inf)
    v, l, pind = attention.partial_attention(b)
    assert list(pind) == [0, 0, 1, 1]
    mo, ml = attention.merge_states(v, l, pind)
    assert np.array_equal(mo[2], np.zeros((2, 8))) and np.all(ml[2] == -np.inf)
    assert np.max(np.abs(mo[1] - out[1])) < 1e-13
