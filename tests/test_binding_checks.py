"""The binding refuses pool and page-table tensors it would otherwise pass
with the wrong layout (no GPU: building the C structs touches no device).
A strided K view such as cache[:, 0] of a [N, 2, Hkv, P, D] tensor would be
read with HND strides, and an int64 page table would be read as int32
words, so both must raise instead."""
import numpy as np
import pytest
import torch

import paged_split_kv_v2_amd as pdk


def pool(k, v=None, dv=8):
    return pdk.KVPool(k=k, v=v, head_dim_v=dv)


def test_contiguous_pool_is_accepted():
    k = torch.zeros(4, 2, 16, 8, dtype=torch.bfloat16)
    s = pool(k, k.clone()).struct()
    assert (s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim_k) == (4, 2, 16, 8)


def test_strided_pool_view_is_refused():
    cache = torch.zeros(4, 2, 2, 16, 8, dtype=torch.bfloat16)  # [N, K/V, Hkv, P, D]
    with pytest.raises(ValueError):
        pool(cache[:, 0], cache[:, 1]).struct()
    k = torch.zeros(4, 2, 16, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pool(k, cache[:, 1]).struct()


def test_pool_shape_and_dtype_mismatches_are_refused():
    k = torch.zeros(4, 2, 16, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pool(k.view(4, 2, 128)).struct()                       # not 4-D
    with pytest.raises(ValueError):
        pool(k, torch.zeros(4, 2, 16, 8, dtype=torch.float32)).struct()
    with pytest.raises(ValueError):
        pool(k, torch.zeros(4, 1, 16, 8, dtype=torch.bfloat16)).struct()
    with pytest.raises(ValueError):
        pool(k, k.clone(), dv=4).struct()                      # v's last dim != head_dim_v


def table(**over):
    t = dict(indptr=torch.tensor([0, 2, 3], dtype=torch.int32),
             indices=torch.tensor([5, 1, 7], dtype=torch.int32),
             kv_len=torch.tensor([20, 9], dtype=torch.int32))
    t.update(over)
    return pdk.DeviceCSR(**t)


def test_int32_table_is_accepted():
    s = table().struct()
    assert (s.batch, s.nnz) == (2, 3)


@pytest.mark.parametrize("name", ["indptr", "indices", "kv_len"])
def test_int64_table_is_refused(name):
    t = table()
    with pytest.raises(ValueError):
        table(**{name: getattr(t, name).to(torch.int64)}).struct()


def test_strided_or_short_table_is_refused():
    wide = torch.tensor([[0, 9], [2, 9], [3, 9]], dtype=torch.int32)
    with pytest.raises(ValueError):
        table(indptr=wide[:, 0]).struct()                      # strided view
    with pytest.raises(ValueError):
        table(indptr=torch.tensor([0, 2], dtype=torch.int32)).struct()  # batch + 1 entries
