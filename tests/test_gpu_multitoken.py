"""Multi-token query steps on the GPU against the oracle: T query tokens per
request, causal over the request's range (token t sees positions up to
kv_len - T + t) or non-causal, on every kernel the row count selects (vector
path up to 16 rows per KV head, matrix-core path above, the small-page
fallback), the flat partial + merge, and the chunked cached-prefix split of
an MLA share with fp8 chunks (non-causal) and a bf16 suffix (causal)
[DCP-PR, section 3.2 figure]. Lengths include ranges shorter than T (query
tokens that see nothing: the empty state) and partitions that end inside
the causal boundary. Pools are NaN-poisoned outside every range."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from oracle import multitoken as omt
from gpu_util import TOL, assert_close, assert_lse, to_device

pytestmark = pytest.mark.gpu


def mt_partials(pdk, b, causal, S):
    pool, csr, q = to_device(b)
    pind = pdk.partition_indptr(b.kv_len, S)
    v, l = pdk.paged_multi_token_partial(pool, csr, q, b.sm_scale, causal, S,
                                         torch.from_numpy(pind).cuda(), int(pind[-1]))
    out, lse = pdk.multi_token_flat(pool, csr, q, b.sm_scale, causal, S,
                                    torch.from_numpy(pind).cuda(), int(pind[-1]))
    torch.cuda.synchronize()
    return v.cpu().numpy(), l.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy(), pind


def check(pdk, b, causal, S):
    v, l, out, lse, pind = mt_partials(pdk, b, causal, S)
    rv, rl, rpind = omt.multi_token_partials(b, causal, S)
    assert np.array_equal(pind, rpind)
    tol = TOL[b.kv_dtype]
    assert_close(v, rv, tol, "multi-token partial out")
    assert_lse(l, rl, "multi-token partial lse")
    ro, rlse = omt.multi_token_attention(b, causal)
    assert_close(out, ro, tol, "multi-token out")
    assert_lse(lse, rlse, "multi-token lse")
    return v, l


# rows per KV head = T * G: 4 / 8 / 16 (vector path), 32 and 64 (matrix cores)
@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("causal", [True, False])
def test_llama_shape_multi_token(gpu, T, causal):
    lens = [T - 1 if T > 1 else 1, T, 17, 63, 64, 65, 300, 1029]
    base = W.random_batch(400 + T, batch=len(lens), page_size=16, num_q_heads=32,
                          num_kv_heads=8, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
                          min_len=0, max_len=0, partition_tokens=64, lens=lens)
    b = W.with_query_tokens(base, T, 410 + T)
    check(gpu, b, causal, 64)


def test_one_token_step_equals_the_decode_entry_point(gpu):
    base = W.llama3_8b_flat(seed=420, batch=5, min_len=50, max_len=900)
    b = W.with_query_tokens(base, 1, 421)
    pool, csr, q = to_device(b)
    S = 128
    pind = gpu.partition_indptr(b.kv_len, S)
    pind_d = torch.from_numpy(pind).cuda()
    v1, l1 = gpu.paged_decode_partial(pool, csr, q[:, 0].contiguous(), b.sm_scale, S, pind_d,
                                      int(pind[-1]))
    for causal in (True, False):
        v, l = gpu.paged_multi_token_partial(pool, csr, q, b.sm_scale, causal, S, pind_d,
                                             int(pind[-1]))
        torch.cuda.synchronize()
        assert torch.equal(v[:, 0], v1) and torch.equal(l[:, 0], l1)


@pytest.mark.parametrize("kv_dtype,T", [("f32", 3), ("bf16", 5)])
def test_other_groupings_and_dtypes(gpu, kv_dtype, T):
    # G = 4 (f32: vector path, 12 rows) and G = 1 (bf16, 5 rows)
    Hq, Hkv = (8, 2) if kv_dtype == "f32" else (4, 4)
    base = W.random_batch(430 + T, batch=6, page_size=8, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=64, kv_dtype=kv_dtype, q_dtype=kv_dtype, min_len=0,
                          max_len=150, partition_tokens=32, lens=[0, 2, 9, 40, 64, 150])
    b = W.with_query_tokens(base, T, 431 + T)
    check(gpu, b, True, 32)


@pytest.mark.parametrize("page_size", [2, 4])
def test_small_pages_matrix_core_paths(gpu, page_size):
    # 32 rows per KV head: pages of 4 take the LDS-ring kernel, pages of 2
    # the register-staged fallback
    base = W.random_batch(440 + page_size, batch=5, page_size=page_size, num_q_heads=32,
                          num_kv_heads=8, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
                          min_len=0, max_len=0, partition_tokens=32, lens=[5, 8, 31, 33, 97])
    b = W.with_query_tokens(base, 8, 441)
    check(gpu, b, True, 32)


def run_mla_mt(pdk, share, staged):
    pre, suf = share.prefix, share.suffix
    p_pool, _, q = to_device(pre)
    s_pool, _, _ = to_device(suf)
    plan = pdk.ChunkedPlan((pre.indptr, pre.indices, pre.kv_len), pre.page_size,
                           share.chunk_tokens, pre.partition_tokens,
                           (suf.indptr, suf.indices, suf.kv_len), suf.page_size,
                           suf.partition_tokens)
    B, T, Hq, Dv = q.shape[0], q.shape[1], q.shape[2], pre.head_dim_v
    co = cl = None
    if staged:
        n = plan.counts()["chunks"]
        co = torch.empty((n, T, Hq, Dv), dtype=torch.float32, device="cuda")
        cl = torch.empty((n, T, Hq), dtype=torch.float32, device="cuda")
    out, lse = plan.run(p_pool, s_pool, q, pre.sm_scale, chunk_out=co, chunk_lse=cl)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("T,page_size", [(2, 64), (4, 64), (3, 16)])
def test_mla_share_multi_token(gpu, T, page_size):
    # 128 heads x T tokens per latent KV head: the latent kernel (pages of
    # 64) or the register-staged fallback (pages of 16)
    share = W.mla_share_with_query_tokens(
        W.mla_decode_share(seed=450 + T, batch=3, context=1024 + 64 * T, suffix_tokens=64 * T,
                           chunk_tokens=512, page_size=page_size, partition_tokens=256,
                           suffix_partition_tokens=32 if page_size == 16 else 64), T, 451)
    ro, rl = omt.mla_multi_token_flat(share)
    for staged in (True, False):
        out, lse = run_mla_mt(gpu, share, staged)
        assert_close(out, ro, TOL["fp8_e4m3"], f"mla multi-token out (staged={staged})")
        assert_lse(lse, rl, f"mla multi-token lse (staged={staged})")


def test_multi_token_repeat_is_deterministic(gpu):
    base = W.random_batch(460, batch=4, page_size=16, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, kv_dtype="bf16", q_dtype="bf16", min_len=0, max_len=0,
                          partition_tokens=64, lens=[3, 70, 129, 500])
    b = W.with_query_tokens(base, 4, 461)
    first = mt_partials(gpu, b, True, 64)
    second = mt_partials(gpu, b, True, 64)
    for x, y in zip(first[:4], second[:4]):
        assert np.array_equal(x, y)


def test_full_size_four_token_step_sampled(gpu):
    """The benchmark's 4-token step at its full size (batch 64, contexts
    U[1024, 8192], 512-token partitions, the launch bench.py times): sampled
    requests against the oracle, every output finite."""
    b = W.with_query_tokens(W.llama3_8b_flat(), 4, 1006)
    pool, csr, q = to_device(b)
    S = b.partition_tokens
    pind = gpu.partition_indptr(b.kv_len, S)
    out, lse = gpu.multi_token_flat(pool, csr, q, b.sm_scale, True, S,
                                    torch.from_numpy(pind).cuda(), int(pind[-1]))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    reqs = [0, 17, 63]
    ro, rl = omt.multi_token_attention(b, True, requests=reqs)
    assert_close(out[reqs], ro[reqs], TOL["bf16"], "4-token out")
    assert_lse(lse[reqs], rl[reqs], "4-token lse")


def test_full_size_four_token_mla_step_sampled(gpu):
    """The benchmark's 4-token MLA step at its full size (batch 32, 128
    heads, 16384 cached fp8 tokens in 4096-token chunks and partitions, 256
    bf16 suffix tokens in one partition, one merge): sampled requests
    against the definition, every output finite."""
    share = W.mla_share_with_query_tokens(
        W.mla_decode_share(partition_tokens=4096, suffix_partition_tokens=256), 4, 1007)
    out, lse = run_mla_mt(gpu, share, staged=False)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    reqs = [0, 21]
    ro, rl = omt.mla_multi_token_flat(share, requests=reqs)
    assert_close(out[reqs], ro[reqs], TOL["fp8_e4m3"], "4-token mla out")
    assert_lse(lse[reqs], rl[reqs], "4-token mla lse")
