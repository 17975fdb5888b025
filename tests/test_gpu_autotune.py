"""Partition autotuning on the GPU [cascade-PR, "What I left out, and where
I was unsure": the shape-bucketed autotuner with cold-L2 methodology]: every
candidate pair is measured, the fastest is kept for the bucket and returned
without measuring on the next call, and the tuned plan's outputs match the
oracle and the flat launch."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from gpu_util import TOL, assert_close, assert_lse, flat_decode, lse_err, rel_err, to_device

pytestmark = pytest.mark.gpu


def test_autotune_picks_the_fastest_and_remembers_the_bucket(gpu):
    gpu.cascade_tuning_clear()
    b = W.cascade_shared_prefix(seed=2300, groups=3, members=6, prefix_tokens=1024,
                                suffix_max=300, extra=3, extra_tokens=700)
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, max_groups=0)
    c0, c1 = [128, 256, 512], [256, 512]
    tuned, info = gpu.cascade_autotune(b.indptr, b.indices, b.kv_len, b.page_size, params, pool,
                                       q, b.sm_scale, c0, c1, reps=2, flush_bytes=64 << 20)
    t = info["times_us"]
    assert info["measured"] and t.shape == (3, 2) and np.all(t > 0)
    i, j = np.unravel_index(np.argmin(t), t.shape)
    assert (tuned.l0_partition_tokens, tuned.l1_partition_tokens) == (c0[i], c1[j])
    assert info["us"] == pytest.approx(float(t[i, j]))
    # same bucket (another seed of the same shape): no measurement
    b2 = W.cascade_shared_prefix(seed=2301, groups=3, members=6, prefix_tokens=1024,
                                 suffix_max=300, extra=3, extra_tokens=700)
    pool2, csr2, q2 = to_device(b2)
    tuned2, info2 = gpu.cascade_autotune(b2.indptr, b2.indices, b2.kv_len, b2.page_size, params,
                                         pool2, q2, b2.sm_scale, c0, c1, reps=2,
                                         flush_bytes=64 << 20)
    assert not info2["measured"] and tuned2 == tuned and np.all(info2["times_us"] == -1)
    looked_up, found = gpu.cascade_tuned_params(b2.indptr, b2.indices, b2.kv_len, b2.page_size,
                                                params, pool2, b2.num_q_heads, gpu.BF16)
    assert found and looked_up == tuned
    # the tuned plan against the oracle and the flat launch
    plan = gpu.CascadePlan(b2.indptr, b2.indices, b2.kv_len, b2.page_size, tuned2)
    out, lse = plan.run(pool2, q2, b2.sm_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = oatt.decode_attention(b2)
    assert_close(out, ro, TOL["bf16"], "tuned cascade out")
    assert_lse(lse, rl, "tuned cascade lse")
    fo, fl, _ = flat_decode(b2, pool2, csr2, q2, 512)
    assert rel_err(out, fo.cpu().numpy()) <= 1e-5
    assert lse_err(lse, fl.cpu().numpy()) <= 1e-5
    gpu.cascade_tuning_clear()


def test_autotune_without_flush_and_declined_plan(gpu):
    gpu.cascade_tuning_clear()
    b = W.llama3_8b_flat(seed=2302, batch=6, min_len=100, max_len=1500)
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1)           # nothing shared: declined, flat
    tuned, info = gpu.cascade_autotune(b.indptr, b.indices, b.kv_len, b.page_size, params, pool,
                                       q, b.sm_scale, [256], [128, 256, 512], reps=1,
                                       flush_bytes=0)
    assert info["measured"] and tuned.l1_partition_tokens in (128, 256, 512)
    plan = gpu.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, tuned)
    assert plan.stats()[1] == "no_candidate"
    out, lse = plan.run(pool, q, b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oatt.decode_attention(b)
    assert_close(out.cpu().numpy(), ro, TOL["bf16"], "tuned flat out")
    assert_lse(lse.cpu().numpy(), rl, "tuned flat lse")
    gpu.cascade_tuning_clear()
