"""Paged split-KV partials and flat decode on the GPU against the oracle
[cascade-PR, "The decomposition" and "How the #898 merge kernel is reused"].

Covers the tiny fp32 workload, the Llama-3-8B-shaped bf16 workload at a
reduced batch (every partial, several tiles, ragged tails) and at its full
size (sampled requests, the launch configuration the benchmark times),
lengths around page and partition boundaries, empty requests, other head
groupings (including more query rows per KV head than one workgroup keeps,
which tiles the rows), and run-to-run determinism. Pools are NaN-poisoned
outside every request's range, so a stray read fails the comparison."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from gpu_util import TOL, assert_close, assert_lse, flat_decode, to_device

pytestmark = pytest.mark.gpu


def partials(pdk, batch, pool, csr, q, S=None):
    S = batch.partition_tokens if S is None else S
    pind = pdk.partition_indptr(batch.kv_len, S)
    v, l = pdk.paged_decode_partial(pool, csr, q, batch.sm_scale, S,
                                    torch.from_numpy(pind).cuda(), int(pind[-1]))
    torch.cuda.synchronize()
    return v.cpu().numpy(), l.cpu().numpy(), pind


def check_partials_and_flat(pdk, batch, S=None):
    pool, csr, q = to_device(batch)
    v, l, pind = partials(pdk, batch, pool, csr, q, S)
    rv, rl, rpind = oatt.partial_attention(batch, S)
    assert np.array_equal(pind, rpind)
    tol = TOL[batch.kv_dtype]
    assert_close(v, rv, tol, "partial out")
    assert_lse(l, rl, "partial lse")
    out, lse, _ = flat_decode(batch, pool, csr, q, S)
    ro, rlse = oatt.decode_attention(batch)
    assert_close(out.cpu().numpy(), ro, tol, "flat out")
    assert_lse(lse.cpu().numpy(), rlse, "flat lse")


def test_tiny_gqa_fp32(gpu):
    check_partials_and_flat(gpu, W.tiny_gqa_fp32())


def test_llama3_shape_reduced_batch(gpu):
    b = W.llama3_8b_flat(seed=2002, batch=6, min_len=100, max_len=1500)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("page_size,S", [(16, 512), (8, 64), (32, 96), (1, 16)])
def test_lengths_around_boundaries(gpu, page_size, S):
    lens = [1, page_size - 1 if page_size > 1 else 1, page_size, page_size + 1, S - 1, S, S + 1,
            2 * S + 3, 0, 7]
    b = W.random_batch(50 + page_size, batch=len(lens), page_size=page_size, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
                       min_len=0, max_len=0, partition_tokens=S, lens=lens)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("Hq,Hkv,D,kv,qd", [
    (8, 8, 128, "bf16", "bf16"),     # G = 1
    (16, 8, 128, "bf16", "bf16"),    # G = 2
    (16, 2, 128, "bf16", "bf16"),    # G = 8
    (32, 2, 64, "f32", "f32"),       # G = 16
    (64, 2, 64, "bf16", "bf16"),     # G = 32: two row tiles per KV head
    (12, 4, 64, "f32", "f32"),       # G = 3 (padded tile)
    (8, 2, 256, "bf16", "bf16"),     # D = 256
    (8, 2, 128, "bf16", "f32"),      # f32 queries on a bf16 pool
    (8, 2, 64, "f32", "bf16"),       # bf16 queries on an f32 pool
    (64, 2, 128, "bf16", "bf16"),    # G = 32: matrix-core tile of 32 rows
    (48, 1, 128, "bf16", "bf16"),    # G = 48: 64-row tile, 16 rows padded
    (160, 1, 128, "bf16", "bf16"),   # G = 160: three 64-row tiles
])
def test_head_groupings_and_dtypes(gpu, Hq, Hkv, D, kv, qd):
    b = W.random_batch(60 + Hq + D, batch=5, page_size=16, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, kv_dtype=kv, q_dtype=qd, min_len=1, max_len=700,
                       partition_tokens=128)
    check_partials_and_flat(gpu, b)


def test_latent_pool_value_aliases_key(gpu):
    # one KV head, V = the key row itself (head_dim_v == head_dim_k here)
    b = W.random_batch(71, batch=4, page_size=16, num_q_heads=8, num_kv_heads=1, head_dim=128,
                       kv_dtype="bf16", q_dtype="bf16", min_len=1, max_len=300,
                       partition_tokens=64, latent=True)
    check_partials_and_flat(gpu, b)


def test_llama3_full_size_sampled(gpu):
    """The benchmark's flat launch: batch 64, lengths U[1024, 8192], 512-token
    partitions. Checked on 6 sampled requests (all heads) and for finiteness
    everywhere."""
    b = W.llama3_8b_flat()
    pool, csr, q = to_device(b)
    out, lse, pind = flat_decode(b, pool, csr, q)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    reqs = [0, 17, 33, int(np.argmax(b.kv_len)), int(np.argmin(b.kv_len)), 63]
    ro, rl = oatt.decode_attention(b, requests=reqs)
    assert_close(out[reqs], ro[reqs], TOL["bf16"], "flat out")
    assert_lse(lse[reqs], rl[reqs], "flat lse")


def test_deterministic(gpu):
    b = W.llama3_8b_flat(seed=2003, batch=8, min_len=500, max_len=3000)
    pool, csr, q = to_device(b)
    o1, l1, _ = flat_decode(b, pool, csr, q)
    o2, l2, _ = flat_decode(b, pool, csr, q)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("page_size", [4, 8, 32, 64])
def test_stacked_rows_page_sizes(gpu, page_size):
    """More than 16 query rows per KV head (the LDS-ring matrix-core path)
    with other page sizes: lengths around page, tile (32 tokens) and
    partition boundaries, one empty request."""
    S = 4 * max(page_size, 32)
    lens = [1, page_size - 1, page_size + 1, 31, 32, 33, S - 1, S, S + 1, 2 * S + 5, 0, 97]
    lens = [max(0, x) for x in lens]
    b = W.random_batch(80 + page_size, batch=len(lens), page_size=page_size, num_q_heads=64,
                       num_kv_heads=2, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
                       min_len=0, max_len=0, partition_tokens=S, lens=lens)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("P,Hkv,Hq,D,Dv,kv,pages", [
    (16, 8, 32, 128, 128, "bf16", 1023),       # vector path
    (16, 2, 32, 128, 128, "bf16", 511),        # LDS-ring path
    (2, 1, 32, 128, 128, "bf16", 1023),        # matrix-core path, 2-token pages
    (64, 1, 128, 576, 512, "fp8_e4m3", 255),   # latent fp8 path
])
def test_largest_partition_each_path_accepts(gpu, P, Hkv, Hq, D, Dv, kv, pages):
    """Partitions of the most pages each kernel stages (one more is refused on
    the host): a request of two such partitions and a ragged tail, one of
    exactly one, one shorter than a page. Partials and flat decode against
    the oracle."""
    S = pages * P
    lens = [2 * S + 37, S, 1]
    b = W.random_batch(4100 + P, batch=3, page_size=P, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, head_dim_v=Dv, kv_dtype=kv, q_dtype="bf16", min_len=0,
                       max_len=0, partition_tokens=S, lens=lens, latent=Dv != D)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("P,Hkv,Hq,D,Dv,kv,base", [
    (16, 8, 32, 128, 128, "bf16", 140_000),        # vector path, 32 KiB pool rows
    (16, 2, 32, 128, 128, "bf16", 600_000),        # LDS-ring path, 8 KiB rows
    (2, 1, 32, 128, 128, "bf16", 9_000_000),       # matrix-core path, 512 B rows
    (64, 1, 128, 576, 512, "fp8_e4m3", 120_000),   # latent fp8 path, 36 KiB rows
])
def test_page_ids_past_4gib_of_pool(gpu, P, Hkv, Hq, D, Dv, kv, base):
    """Every page a request reads lies more than 4 GiB (and more than 2^31
    elements) into its pool: the same rows as a small pool, moved up by
    `base` rows of a large one, with the page ids moved by the same amount.
    Partials and flat decode against the oracle on the small pool."""
    b = W.random_batch(4200 + P, batch=3, page_size=P, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, head_dim_v=Dv, kv_dtype=kv, q_dtype="bf16", min_len=1,
                       max_len=900, partition_tokens=256, latent=Dv != D)
    small, _, q = to_device(b)

    def lift(t):
        big = torch.empty((base + t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype,
                          device=t.device)
        big[base:] = t
        return big

    pool = gpu.KVPool(k=lift(small.k), v=None if small.v is None else lift(small.v),
                      head_dim_v=small.head_dim_v, k_scale=small.k_scale, v_scale=small.v_scale)
    assert pool.k.numel() * pool.k.element_size() > 4 << 30
    assert base * pool.k[0].numel() > 2**31
    csr = gpu.DeviceCSR.from_host(b.indptr, b.indices + base, b.kv_len)
    v, l, pind = partials(gpu, b, pool, csr, q)
    rv, rl, _ = oatt.partial_attention(b)
    tol = TOL[b.kv_dtype]
    assert_close(v, rv, tol, "partial out")
    assert_lse(l, rl, "partial lse")
    out, lse, _ = flat_decode(b, pool, csr, q)
    ro, rlse = oatt.decode_attention(b)
    assert_close(out.cpu().numpy(), ro, tol, "flat out")
    assert_lse(lse.cpu().numpy(), rlse, "flat lse")


def test_many_short_requests(gpu):
    """2,000 requests of 0-70 tokens (empty ones included) in 32-token
    partitions: the request search over a long batch, many partitions and
    merge groups of every small size. Partials and flat decode against the
    oracle."""
    b = W.random_batch(4300, batch=2000, page_size=16, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, kv_dtype="bf16", q_dtype="bf16", min_len=0, max_len=70,
                       partition_tokens=32)
    assert (b.kv_len == 0).any() and b.kv_len.max() > 64
    check_partials_and_flat(gpu, b)


def test_every_request_empty(gpu):
    """A batch whose requests all have no tokens: no partitions, no partial
    launch; the merge alone writes out = 0 and lse = -inf for every row (the
    oracle's empty state), through decode_flat and decode_flat_noalloc."""
    b = W.random_batch(4400, batch=5, page_size=16, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, kv_dtype="bf16", q_dtype="bf16", min_len=0, max_len=0,
                       partition_tokens=64, lens=[0] * 5)
    pool, csr, q = to_device(b)
    pind = gpu.partition_indptr(b.kv_len, 64)
    assert int(pind[-1]) == 0
    ro, rl = oatt.decode_attention(b)
    assert np.all(ro == 0) and np.all(rl == -np.inf)
    out, lse, _ = flat_decode(b, pool, csr, q, 64)
    assert np.all(out.cpu().numpy() == 0) and np.all(lse.cpu().numpy() == -np.inf)
    out2 = torch.full_like(out, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    gpu.decode_flat_noalloc(pool, csr, q, b.sm_scale, 64, torch.from_numpy(pind).cuda(), 0, out2,
                            lse2)
    torch.cuda.synchronize()
    assert np.all(out2.cpu().numpy() == 0) and np.all(lse2.cpu().numpy() == -np.inf)
