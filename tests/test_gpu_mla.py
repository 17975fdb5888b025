"""Chunked cached-prefix + new-suffix decode of an MLA share on the GPU
[DCP-PR, section 3.2 figure: each cached-prefix chunk returns (O, LSE); the
chunk states are LSE-merged, then merged with the new-token suffix state;
3.3: fp8 rows are dequantized to bf16 with the per-tensor scale].

Checked against the oracle's chunk states and against the plain definition
(one softmax over prefix and suffix tokens), tolerance 5e-3 (fp8 KV after the
identical dequant), LSE within 1e-4. Without chunk outputs the library merges
all partials of a request in one launch; that regrouping is checked against
the staged merges to 1e-5 [cascade-PR, "How the #898 merge kernel is reused":
merging is associative]."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import mla as omla
from gpu_util import TOL, assert_close, assert_lse, to_device

pytestmark = pytest.mark.gpu


def run_chunked(pdk, share, staged=True):
    """staged: with per-chunk outputs (the staged merges); else one merge."""
    pre, suf = share.prefix, share.suffix
    p_pool, _, q = to_device(pre)
    s_pool, _, _ = to_device(suf)
    plan = pdk.ChunkedPlan((pre.indptr, pre.indices, pre.kv_len), pre.page_size,
                           share.chunk_tokens, pre.partition_tokens,
                           (suf.indptr, suf.indices, suf.kv_len), suf.page_size,
                           suf.partition_tokens)
    counts = plan.counts()
    Hq, Dv = pre.num_q_heads, pre.head_dim_v
    if not staged:
        out, lse = plan.run(p_pool, s_pool, q, pre.sm_scale)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), None, None, counts
    chunk_out = torch.empty((counts["chunks"], Hq, Dv), dtype=torch.float32, device="cuda")
    chunk_lse = torch.empty((counts["chunks"], Hq), dtype=torch.float32, device="cuda")
    out, lse = plan.run(p_pool, s_pool, q, pre.sm_scale, chunk_out=chunk_out,
                        chunk_lse=chunk_lse)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), lse.cpu().numpy(), chunk_out.cpu().numpy(),
            chunk_lse.cpu().numpy(), counts)


@pytest.mark.parametrize("context,chunk,part,spart", [(2048, 1024, 512, 64), (1000, 512, 256, 128),
                                                     (4096, 4096, 2048, 64)])
def test_mla_share_small(gpu, context, chunk, part, spart):
    share = W.mla_decode_share(seed=3005, batch=3, heads=128, context=context,
                               suffix_tokens=100, chunk_tokens=chunk, partition_tokens=part,
                               suffix_partition_tokens=spart)
    out, lse, cout, clse, counts = run_chunked(gpu, share)
    assert counts["chunks"] == 3 * -(-context // chunk)
    ro, rl, rco, rcl = omla.mla_decode(share)
    assert_close(cout, rco, TOL["fp8_e4m3"], "chunk out")
    assert_lse(clse, rcl, "chunk lse")
    assert_close(out, ro, TOL["fp8_e4m3"], "out")
    assert_lse(lse, rl, "lse")
    fo, fl = omla.mla_flat(share)
    assert_close(out, fo, TOL["fp8_e4m3"], "out vs one softmax")
    # one merge over all partials of a request = the staged merges
    o1, l1, _, _, _ = run_chunked(gpu, share, staged=False)
    assert_close(o1, out, 1e-5, "single merge vs staged")
    assert np.max(np.abs(l1 - lse)) <= 1e-5


def test_mla_share_full_size_sampled(gpu):
    """Batch 32, 128 heads, 16384 cached fp8 tokens in 4096-token chunks plus
    256 bf16 suffix tokens, in the launch configuration the benchmark times
    (2048-token partitions, 64-token suffix partitions, one merge): sampled
    requests against the definition."""
    share = W.mla_decode_share()
    out, lse, _, _, counts = run_chunked(gpu, share, staged=False)
    assert counts["chunks"] == 32 * 4
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    reqs = [0, 13, 31]
    fo, fl = omla.mla_flat(share, requests=reqs)
    assert_close(out[reqs], fo[reqs], TOL["fp8_e4m3"], "out")
    assert_lse(lse[reqs], fl[reqs], "lse")


def test_mla_ragged_and_empty_suffix(gpu):
    """Contexts shorter than one chunk, not a multiple of the tile or page,
    and requests whose new-token suffix is empty (their state is the prefix
    state alone)."""
    pre_lens, suf_lens = [100, 1024 + 37, 64, 5], [0, 70, 128, 0]
    pre = W.random_batch(3101, batch=4, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="fp8_e4m3", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=256, lens=pre_lens, latent=True)
    suf = W.random_batch(3102, batch=4, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="bf16", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=64, lens=suf_lens, latent=True)
    suf.q = pre.q
    suf.sm_scale = pre.sm_scale
    share = W.MlaShare(prefix=pre, suffix=suf, chunk_tokens=512)
    out, lse, cout, clse, counts = run_chunked(gpu, share)
    ro, rl, rco, rcl = omla.mla_decode(share)
    assert_close(cout, rco, TOL["fp8_e4m3"], "chunk out")
    assert_lse(clse, rcl, "chunk lse")
    assert_close(out, ro, TOL["fp8_e4m3"], "out")
    assert_lse(lse, rl, "lse")
    fo, fl = omla.mla_flat(share)
    assert_close(out, fo, TOL["fp8_e4m3"], "out vs one softmax")
    o1, l1, _, _, _ = run_chunked(gpu, share, staged=False)
    assert_close(o1, out, 1e-5, "single merge vs staged")


def test_mla_partitions_of_every_tile_count_mod_three(gpu):
    """Partitions of 3, 5, 6 and 9 tiles of 32 tokens (and a suffix of 3, 4, 2
    and 1 tiles): the bf16 latent kernel cycles three tile buffers and the
    fp8 one two, so the last tile of a partition sits in every buffer across
    these cases."""
    pre_lens, suf_lens = [96, 150, 190, 288], [96, 0, 190, 32]
    pre = W.random_batch(3111, batch=4, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="fp8_e4m3", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=512, lens=pre_lens, latent=True)
    suf = W.random_batch(3112, batch=4, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="bf16", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=128, lens=suf_lens, latent=True)
    suf.q = pre.q
    suf.sm_scale = pre.sm_scale
    share = W.MlaShare(prefix=pre, suffix=suf, chunk_tokens=512)
    out, lse, cout, clse, counts = run_chunked(gpu, share)
    ro, rl, rco, rcl = omla.mla_decode(share)
    assert_close(cout, rco, TOL["fp8_e4m3"], "chunk out")
    assert_lse(clse, rcl, "chunk lse")
    assert_close(out, ro, TOL["fp8_e4m3"], "out")
    assert_lse(lse, rl, "lse")


def test_mla_scores_far_above_the_first_tile(gpu):
    """The fp8 latent kernel exponentiates against each row's first-tile
    maximum and restarts the partition with a raised reference when a later
    score exceeds it by more than 2^16; these keys force that: request 0 has
    one key aligned with head 0's query in its fourth tile (one restart),
    request 1 one in its second tile and a larger one in its eighth (two
    restarts), request 2 is untouched. Against the one-softmax definition."""
    pre_lens, suf_lens = [512, 300, 700], [40, 0, 64]
    pre = W.random_batch(3121, batch=3, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="fp8_e4m3", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=512, lens=pre_lens, latent=True)
    suf = W.random_batch(3122, batch=3, page_size=64, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, head_dim_v=512, kv_dtype="bf16", q_dtype="bf16",
                         min_len=0, max_len=0, partition_tokens=64, lens=suf_lens, latent=True)
    suf.q = pre.q
    suf.sm_scale = pre.sm_scale
    qf = (pre.q.astype(np.uint32) << 16).view(np.float32)  # bf16 bits -> f32
    for b, t, amp in ((0, 100, 1.0), (1, 40, 0.8), (1, 250, 2.0)):
        row = int(pre.indices[pre.indptr[b] + t // 64])
        key = amp * np.sign(qf[b, 0]).astype(np.float32)
        pre.k_pool[row, 0, t % 64] = W._fp8_bits(key, pre.k_scale)
    share = W.MlaShare(prefix=pre, suffix=suf, chunk_tokens=512)
    out, lse, _, _, _ = run_chunked(gpu, share, staged=False)
    fo, fl = omla.mla_flat(share)
    # the planted keys do dominate head 0 of the requests that hold them
    s = fl[:2, 0] - np.delete(fl[:2], 0, axis=1).max(axis=1)
    assert np.all(s > 10), s
    assert_close(out, fo, TOL["fp8_e4m3"], "out")
    assert_lse(lse, fl, "lse")


@pytest.mark.parametrize("Hq,kv", [(128, "fp8_e4m3"), (80, "fp8_e4m3"), (128, "bf16")])
def test_latent_shared_prefix_stacked(gpu, Hq, kv):
    """A shared-prefix cascade over a latent pool [cascade-PR, "The
    decomposition"]: the shared span's level-0 launch stacks three members'
    query rows (three row tiles at 128 heads), so the latent kernels take
    each wave's query rows from one member's slot; at 80 heads a wave's rows
    straddle two members. Against the one-softmax definition per request."""
    from oracle import attention as oatt
    lens = [700, 450, 520, 300]
    b = W.random_batch(3131, batch=4, page_size=64, num_q_heads=Hq, num_kv_heads=1,
                       head_dim=576, head_dim_v=512, kv_dtype=kv, q_dtype="bf16",
                       min_len=0, max_len=0, partition_tokens=256, lens=lens,
                       share=[([0, 1, 2], 6)], latent=True)
    pool, _, q = to_device(b)
    plan = gpu.CascadePlan(b.indptr, b.indices, b.kv_len, 64,
                           gpu.CascadeParams(enabled=1, min_shared_pages=2,
                                             l0_partition_tokens=256, l1_partition_tokens=256))
    out, lse = plan.run(pool, q, b.sm_scale)
    torch.cuda.synchronize()
    assert plan.stats()[0]["members"] == 3
    ro, rl = oatt.decode_attention(b)
    assert_close(out.cpu().numpy(), ro, TOL[kv], "out")
    assert_lse(lse.cpu().numpy(), rl, "lse")


def test_latent_fp8_80_query_heads(gpu):
    """80 query heads on one latent KV head: the third wave of a workgroup
    holds 16 live rows and the fourth none. Partials and flat decode against
    the oracle."""
    from test_gpu_partial import check_partials_and_flat
    b = W.random_batch(3132, batch=3, page_size=64, num_q_heads=80, num_kv_heads=1,
                       head_dim=576, head_dim_v=512, kv_dtype="fp8_e4m3", q_dtype="bf16",
                       min_len=1, max_len=700, partition_tokens=256, latent=True)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("P,lens", [
    (64, [4096, 4096, 4090, 4101]),   # >= 256 partitions: 8-wave, 128-row workgroups
    (64, [300, 129, 64, 1, 0]),       # a small grid: 4-wave, 64-row workgroups
    (16, [300, 129, 64, 1, 0]),       # pages under 32 tokens: the 16-row matrix-core kernel
])
def test_latent_bf16_partials_at_the_bf16_bar(gpu, P, lens):
    """bf16 latent pools (the MLA new-token range, or a bf16 cached prefix)
    through each kernel that reads them, in 64-token partitions (ragged
    last ones, an empty request): partials and flat decode against the
    oracle at the bf16 bar, which needs P carried as bf16 hi + lo."""
    from test_gpu_partial import check_partials_and_flat
    b = W.random_batch(3133, batch=len(lens), page_size=P, num_q_heads=128, num_kv_heads=1,
                       head_dim=576, head_dim_v=512, kv_dtype="bf16", q_dtype="bf16",
                       min_len=0, max_len=0, partition_tokens=64, lens=lens, latent=True)
    check_partials_and_flat(gpu, b)


@pytest.mark.parametrize("seed", range(6))
def test_latent_fp8_short_partitions(gpu, seed):
    """Many short fp8 partitions (24 requests of 1-63 tokens, one 64-token
    partition each, 128 heads): where one or two tokens carry a row's
    weight, the fp8 kernel's single bf16 rounding of P is least averaged
    out. Partials and flat decode against the oracle at the fp8 bar."""
    from test_gpu_partial import check_partials_and_flat
    lens = [int(x) for x in np.random.default_rng(seed).integers(1, 64, size=24)]
    b = W.random_batch(5000 + seed, batch=24, page_size=64, num_q_heads=128, num_kv_heads=1,
                       head_dim=576, head_dim_v=512, kv_dtype="fp8_e4m3", q_dtype="bf16",
                       min_len=0, max_len=0, partition_tokens=64, lens=lens, latent=True)
    check_partials_and_flat(gpu, b)
