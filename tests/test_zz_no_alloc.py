"""pdk_decode_flat_noalloc (partial states in the library's static device
array, no workspace) through the C ABI against pdk_decode_flat (caller
workspace) on the same inputs: two calls in a row, the second on a smaller
batch, so the second reads an array still holding the first call's states;
both also against the f64 oracle on sampled requests (bf16 KV, 2e-3;
LSE 1e-4 log2 units). A call whose states exceed the array is refused
before any launch."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from gpu_util import TOL, assert_close, assert_lse, lse_err, rel_err, to_device

pytestmark = pytest.mark.gpu


def run_both(pdk, b, S):
    pool, csr, q = to_device(b)
    pind = pdk.partition_indptr(b.kv_len, S)
    pind_d = torch.from_numpy(pind).cuda()
    R = int(pind[-1])
    ref_o, ref_l = pdk.decode_flat(pool, csr, q, b.sm_scale, S, pind_d, R)
    out = torch.full((b.batch, b.num_q_heads, b.head_dim_v), float("nan"), device="cuda")
    lse = torch.full((b.batch, b.num_q_heads), float("nan"), device="cuda")
    pdk.decode_flat_noalloc(pool, csr, q, b.sm_scale, S, pind_d, R, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), ref_o.cpu().numpy(), ref_l.cpu().numpy()


def check(b, got, sample):
    out, lse, ref_o, ref_l = got
    # against the workspace entry point: same kernels, GPU vs GPU bar
    assert rel_err(out, ref_o) <= 1e-5 and lse_err(lse, ref_l) <= 1e-5
    ro, rl = oatt.decode_attention(b, requests=sample)
    assert_close(out[sample], ro[sample], TOL[b.kv_dtype], "noalloc out")
    assert_lse(lse[sample], rl[sample], "noalloc lse")


def test_two_calls_second_smaller(gpu):
    big = W.llama3_8b_flat()                      # 64 requests, 512-token partitions
    got = run_both(gpu, big, big.partition_tokens)
    check(big, got, [0, 17, 63])
    small = W.llama3_8b_flat(seed=2003, batch=5, min_len=40, max_len=700)
    got = run_both(gpu, small, 256)
    check(small, got, list(range(5)))


def test_states_beyond_the_array_are_refused(gpu):
    b = W.llama3_8b_flat(seed=2004, batch=2, min_len=64, max_len=64)
    pool, csr, q = to_device(b)
    per_part = b.num_q_heads * (b.head_dim_v + 1) * 4
    R = gpu.DECODE_FLAT_NOALLOC_MAX_BYTES // per_part + 1
    pind = torch.zeros(b.batch + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((b.batch, b.num_q_heads, b.head_dim_v), device="cuda")
    with pytest.raises(gpu.PdkError) as e:
        gpu.decode_flat_noalloc(pool, csr, q, b.sm_scale, 64, pind, R, out)
    assert e.value.status == -5  # PDK_ERR_WORKSPACE, refused before any launch
