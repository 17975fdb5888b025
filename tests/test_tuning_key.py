"""Shape buckets of the partition autotuner (host only, no GPU): steps that
differ only within a bucket share tuned sizes, steps whose shapes differ do
not [cascade-PR, "What I left out, and where I was unsure": a shape-bucketed
autotuner for the cascade levels]."""
import numpy as np
import pytest
import torch

import paged_split_kv_v2_amd as pdk
import workloads as W


def pool_of(b):
    # host tensors stand in for the pool: the key reads shapes and dtypes only
    k = torch.from_numpy(b.k_pool.view(np.int16)).view(torch.bfloat16)
    v = torch.from_numpy(b.v_pool.view(np.int16)).view(torch.bfloat16)
    return pdk.KVPool(k=k, v=v, head_dim_v=b.head_dim_v)


P = pdk.CascadeParams(enabled=1, max_groups=0)


def key(b, params=P, Hq=None):
    return pdk.cascade_tuning_key(b.indptr, b.indices, b.kv_len, b.page_size, params, pool_of(b),
                                  b.num_q_heads if Hq is None else Hq, pdk.BF16)


def test_same_shape_other_seed_shares_the_bucket():
    a = W.cascade_shared_prefix(seed=2200, groups=3, members=6, prefix_tokens=1024,
                                suffix_max=300, extra=3, extra_tokens=700)
    b = W.cascade_shared_prefix(seed=2201, groups=3, members=6, prefix_tokens=1024,
                                suffix_max=300, extra=3, extra_tokens=700)
    assert not np.array_equal(a.kv_len, b.kv_len)
    assert key(a) == key(b)


def test_shapes_that_matter_change_the_bucket():
    base = W.cascade_shared_prefix(seed=2202, groups=3, members=6, prefix_tokens=1024,
                                   suffix_max=300, extra=3, extra_tokens=700)
    k0 = key(base)
    longer = W.cascade_shared_prefix(seed=2202, groups=3, members=6, prefix_tokens=4096,
                                     suffix_max=300, extra=3, extra_tokens=700)
    assert key(longer) != k0                   # shared and total tokens
    bigger = W.cascade_shared_prefix(seed=2202, groups=6, members=12, prefix_tokens=1024,
                                     suffix_max=300, extra=3, extra_tokens=700)
    assert key(bigger) != k0                   # batch and members
    assert key(base, Hq=64) != k0              # query heads per KV head
    assert key(base, params=pdk.CascadeParams(enabled=1, max_groups=1)) != k0
    assert key(base, params=pdk.CascadeParams(enabled=0)) != k0   # declined plan
    # the partition sizes themselves are what is tuned, not part of the key
    assert key(base, params=pdk.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=512,
                                              l1_partition_tokens=1024)) == k0


def test_untuned_bucket_keeps_the_given_sizes():
    pdk.cascade_tuning_clear()
    b = W.cascade_shared_prefix(seed=2203, groups=2, members=4, prefix_tokens=512,
                                suffix_max=200, extra=1, extra_tokens=300)
    tuned, found = pdk.cascade_tuned_params(b.indptr, b.indices, b.kv_len, b.page_size, P,
                                            pool_of(b), b.num_q_heads, pdk.BF16)
    assert not found and tuned == P


def test_bad_candidates_are_rejected():
    b = W.cascade_shared_prefix(seed=2204, groups=2, members=4, prefix_tokens=512,
                                suffix_max=200, extra=1, extra_tokens=300)
    s, keep = pdk._host_csr(b.indptr, b.indices, b.kv_len)
    p = P.struct()
    c, cp = pdk._i32([256, 24])               # 24 is not a multiple of 16
    import ctypes
    assert pdk.lib().pdk_cascade_autotune_workspace_bytes(ctypes.byref(s), 16, ctypes.byref(p),
                                                          cp, 2, cp, 1, 32, 128) == 0
