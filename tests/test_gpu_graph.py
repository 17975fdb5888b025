"""Step graphs on the GPU: a decode step's launches recorded once by HIP
stream capture and replayed. Each graph holds kernel nodes only; every
replay, with eager work and synchronizations between replays, equals the
eager run of the same step bit for bit (the same kernels with the same
arguments); a replay after the queries change in place equals an eager run
on the new queries; the replayed outputs are also checked against the
oracle. Shapes: a shared-prefix cascade, the chunked MLA share, and the
flat decode without a workspace."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from oracle import mla as omla
from gpu_util import TOL, assert_close, assert_lse, dev_tensor, to_device

pytestmark = pytest.mark.gpu


def replays_equal(graph, outs, want, between):
    """Three replays, each after `between()` (eager work that overwrites the
    outputs) and a synchronization; every replay equals `want` bit for bit."""
    for _ in range(3):
        between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref)


def scramble(*ts):
    def f():
        for t in ts:
            t.fill_(float("nan"))
    return f


def test_cascade_step_graph(gpu):
    b = W.cascade_shared_prefix(seed=2601, groups=2, members=4, prefix_tokens=512,
                                suffix_min=20, suffix_max=300, extra=2, extra_tokens=700)
    pool, _, q = to_device(b)
    plan = gpu.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size,
                           gpu.CascadeParams(enabled=1, min_shared_pages=2,
                                             l0_partition_tokens=256, l1_partition_tokens=256))
    Hq, Dv = b.num_q_heads, b.head_dim_v
    plan.upload(Hq, Dv, q.device)
    eo, el = plan.run(pool, q, b.sm_scale)
    out = torch.empty_like(eo)
    lse = torch.empty_like(el)
    g = gpu.StepGraph(lambda: plan.run(pool, q, b.sm_scale, out, lse))
    kernels, others = g.node_counts()
    assert kernels >= 2 and others == 0, (kernels, others)
    replays_equal(g, (out, lse), (eo, el), scramble(out, lse))
    ro, rl = oatt.decode_attention(b)
    assert_close(out.cpu().numpy(), ro, TOL["bf16"], "replayed out")
    assert_lse(lse.cpu().numpy(), rl, "replayed lse")
    # new queries in place: the replay reads them
    q2 = W.random_batch(2602, batch=b.batch, page_size=b.page_size, num_q_heads=Hq,
                        num_kv_heads=b.num_kv_heads, head_dim=b.head_dim_k, kv_dtype="bf16",
                        q_dtype="bf16", min_len=1, max_len=1, partition_tokens=256).q
    q.copy_(dev_tensor(q2))
    eo2, el2 = plan.run(pool, q, b.sm_scale)
    replays_equal(g, (out, lse), (eo2, el2), scramble(out, lse))
    assert not torch.equal(eo2, eo)


def test_chunked_mla_step_graph(gpu):
    share = W.mla_decode_share(seed=2603, batch=3, heads=128, context=1000, suffix_tokens=100,
                               chunk_tokens=512, partition_tokens=256, suffix_partition_tokens=64)
    pre, suf = share.prefix, share.suffix
    p_pool, _, q = to_device(pre)
    s_pool, _, _ = to_device(suf)
    plan = gpu.ChunkedPlan((pre.indptr, pre.indices, pre.kv_len), pre.page_size,
                           share.chunk_tokens, pre.partition_tokens,
                           (suf.indptr, suf.indices, suf.kv_len), suf.page_size,
                           suf.partition_tokens)
    Hq, Dv = pre.num_q_heads, pre.head_dim_v
    plan.upload(Hq, Dv, q.device)
    out = torch.empty((pre.batch, Hq, Dv), dtype=torch.float32, device=q.device)
    lse = torch.empty((pre.batch, Hq), dtype=torch.float32, device=q.device)
    eo, el = plan.run(p_pool, s_pool, q, pre.sm_scale)
    g = gpu.StepGraph(lambda: plan.run(p_pool, s_pool, q, pre.sm_scale, out, lse))
    kernels, others = g.node_counts()
    assert kernels >= 3 and others == 0, (kernels, others)
    replays_equal(g, (out, lse), (eo, el), scramble(out, lse))
    fo, fl = omla.mla_flat(share)
    assert_close(out.cpu().numpy(), fo, TOL["fp8_e4m3"], "replayed out")
    assert_lse(lse.cpu().numpy(), fl, "replayed lse")


def test_flat_noalloc_step_graph(gpu):
    b = W.llama3_8b_flat(seed=2604, batch=5, min_len=100, max_len=1500)
    pool, csr, q = to_device(b)
    S = b.partition_tokens
    pind = gpu.partition_indptr(b.kv_len, S)
    pind_d = torch.from_numpy(pind).to(q.device)
    R = int(pind[-1])
    shape = (b.batch, b.num_q_heads)
    eo = torch.empty(shape + (b.head_dim_v,), dtype=torch.float32, device=q.device)
    el = torch.empty(shape, dtype=torch.float32, device=q.device)
    gpu.decode_flat_noalloc(pool, csr, q, b.sm_scale, S, pind_d, R, eo, el)
    out, lse = torch.empty_like(eo), torch.empty_like(el)
    g = gpu.StepGraph(lambda: gpu.decode_flat_noalloc(pool, csr, q, b.sm_scale, S, pind_d, R,
                                                      out, lse))
    kernels, others = g.node_counts()
    assert kernels >= 2 and others == 0, (kernels, others)
    replays_equal(g, (out, lse), (eo, el), scramble(out, lse))
    ro, rl = oatt.decode_attention(b)
    assert_close(out.cpu().numpy(), ro, TOL["bf16"], "replayed out")
    assert_lse(lse.cpu().numpy(), rl, "replayed lse")
