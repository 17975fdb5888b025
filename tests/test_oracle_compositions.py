"""Pins for the oracle's cascade and MLA compositions (no GPU).

Both compositions are exact rewrites of full attention, so each is pinned to
the flat definition [cascade-PR, "The decomposition": disjoint key ranges
merge exactly; DCP-PR section 3.2: chunk states merged across chunks and with
the suffix]. The member-major stacking is the negative control
[cascade-PR, "The decomposition"].
"""
import numpy as np

from oracle import attention, cascade, mla, planner
from oracle.planner import CascadeParams
from workloads import (cascade_shared_prefix, mla_decode_share, random_batch,
                       tiny_gqa_fp32)


def test_tiny_cascade_equals_flat():
    b = tiny_gqa_fp32()
    params = CascadeParams(enabled=1, min_shared_pages=2, l0_partition_tokens=32,
                           l1_partition_tokens=32)
    out, lse, plan = cascade.cascade_decode(b, params, return_plan=True)
    assert plan.stats["members"] == 3
    fo, fl = attention.decode_attention(b)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12


def test_member_major_stacking_reads_the_wrong_kv_head():
    b = tiny_gqa_fp32()
    params = CascadeParams(enabled=1, min_shared_pages=2, l0_partition_tokens=32,
                           l1_partition_tokens=32)
    out, _ = cascade.cascade_decode(b, params, head_map_fn=planner.member_major_head_map)
    fo, _ = attention.decode_attention(b)
    assert np.max(np.abs(out - fo)) > 1e-2


def test_random_cascade_equals_flat_all_groups():
    b = random_batch(31, batch=7, page_size=8, num_q_heads=8, num_kv_heads=2, head_dim=16,
                     kv_dtype="bf16", q_dtype="bf16", min_len=40, max_len=70,
                     partition_tokens=16, share=[([0, 2, 3], 4), ([4, 6], 3)])
    params = CascadeParams(enabled=1, min_shared_pages=2, max_groups=0,
                           l0_partition_tokens=16, l1_partition_tokens=24)
    out, lse, plan = cascade.cascade_decode(b, params, return_plan=True)
    assert len(plan.groups) == 2
    fo, fl = attention.decode_attention(b)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12


def test_cascade_workload_small_equals_flat():
    b = cascade_shared_prefix(groups=2, members=3, prefix_tokens=64, suffix_max=80,
                              extra=1, extra_tokens=48)
    b.num_q_heads, b.num_kv_heads = 32, 8
    params = CascadeParams(enabled=1, min_shared_pages=2, max_groups=0,
                           l0_partition_tokens=32, l1_partition_tokens=64)
    reqs = list(range(len(b.kv_len)))
    out, lse = cascade.cascade_decode(b, params)
    fo, fl = attention.decode_attention(b, requests=reqs)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12


def test_mla_chunked_composition_equals_flat():
    share = mla_decode_share(batch=2, heads=4, context=512, suffix_tokens=64,
                             chunk_tokens=128, page_size=64, partition_tokens=64)
    out, lse, chunk_out, chunk_lse = mla.mla_decode(share)
    assert chunk_out.shape[0] == 2 * 4
    fo, fl = mla.mla_flat(share)
    assert np.max(np.abs(out - fo)) < 1e-12 and np.max(np.abs(lse - fl)) < 1e-12
    assert np.all(np.isfinite(out))


def test_mla_value_is_the_first_512_latent_lanes():
    share = mla_decode_share(batch=1, heads=2, context=128, suffix_tokens=64,
                             chunk_tokens=128, page_size=64, partition_tokens=64)
    pre = share.prefix
    K, V = attention.gather(pre.k_pool, pre.v_pool, pre.kv_dtype, pre.k_scale, pre.v_scale,
                            pre.indptr, pre.indices, pre.kv_len, pre.page_size, 0, 512)
    assert K.shape[2] == 576 and V.shape[2] == 512
    assert np.array_equal(V, K[:, :, :512])
