"""Cascade (shared-prefix) decode on the GPU [cascade-PR, "The decomposition",
"Task items" 1-4, "Correctness coverage"]: against the oracle's flat
attention (the exact result the cascade reaches), against the GPU flat path
(1e-5), the declined plan falling back to flat, the single merge against the
page's two-stage form (level merge, then pair merge), the head stack /
unstack kernels, and the member-major negative control."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as oatt
from oracle import planner as oplan
from gpu_util import TOL, assert_close, assert_lse, flat_decode, lse_err, rel_err, to_device

pytestmark = pytest.mark.gpu


def cascade(pdk, batch, params, pool=None, q=None):
    plan = pdk.CascadePlan(batch.indptr, batch.indices, batch.kv_len, batch.page_size, params)
    out, lse = plan.run(pool, q, batch.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), plan


def test_tiny_cascade(gpu):
    b = W.tiny_gqa_fp32()
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, min_shared_pages=2, l0_partition_tokens=32,
                               l1_partition_tokens=32)
    out, lse, plan = cascade(gpu, b, params, pool, q)
    stats, decline = plan.stats()
    assert decline == "none" and stats["members"] == 3 and stats["shared_pages"] == 2
    ro, rl = oatt.decode_attention(b)
    assert_close(out, ro, TOL["f32"], "cascade out")
    assert_lse(lse, rl, "cascade lse")
    fo, fl, _ = flat_decode(b, pool, csr, q, 32)
    assert rel_err(out, fo.cpu().numpy()) <= 1e-5
    assert lse_err(lse, fl.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("max_groups", [1, 0])
def test_cascade_workload_reduced(gpu, max_groups):
    b = W.cascade_shared_prefix(seed=2004, groups=3, members=5, prefix_tokens=1024,
                                suffix_max=400, extra=3, extra_tokens=700)
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, max_groups=max_groups, l0_partition_tokens=256,
                               l1_partition_tokens=512)
    out, lse, plan = cascade(gpu, b, params, pool, q)
    stats, decline = plan.stats()
    assert decline == "none" and stats["members"] == (5 if max_groups == 1 else 15)
    ro, rl = oatt.decode_attention(b)
    assert_close(out, ro, TOL["bf16"], "cascade out")
    assert_lse(lse, rl, "cascade lse")
    fo, fl, _ = flat_decode(b, pool, csr, q, 512)
    assert rel_err(out, fo.cpu().numpy()) <= 1e-5
    assert lse_err(lse, fl.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("case", ["reduced", "ragged"])
def test_fused_levels_equal_two_launches(gpu, case):
    """Levels 0 and 1 in one grid (bf16 pool, head dim 128, 4 query heads
    per KV head: the fused kernel's shape) write the same partial rows as the
    two launches, so the outputs agree bit for bit; both against the oracle."""
    if case == "reduced":
        b = W.cascade_shared_prefix(seed=2006, groups=3, members=6, prefix_tokens=1024,
                                    suffix_max=300, extra=4, extra_tokens=500)
        s0, s1 = 256, 512
    else:  # one-token suffixes, short extras, partitions that end mid-step
        b = W.cascade_shared_prefix(seed=2007, groups=2, members=5, prefix_tokens=528,
                                    suffix_min=1, suffix_max=90, extra=3, extra_tokens=17)
        s0, s1 = 64, 48
    pool, csr, q = to_device(b)
    res = {}
    for fuse in (1, 0):
        params = gpu.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=s0,
                                   l1_partition_tokens=s1, fuse_levels=fuse)
        out, lse, plan = cascade(gpu, b, params, pool, q)
        assert plan.stats()[1] == "none" and plan.stats()[0]["members"] > 4
        res[fuse] = (out, lse)
    assert np.array_equal(res[1][0], res[0][0]) and np.array_equal(res[1][1], res[0][1])
    ro, rl = oatt.decode_attention(b)
    assert_close(res[1][0], ro, TOL["bf16"], "fused cascade out")
    assert_lse(res[1][1], rl, "fused cascade lse")


def test_cached_plan_runs_like_a_fresh_one(gpu):
    """Plans from the plan cache (one per page table, reused by every layer)
    give the same outputs as freshly built plans, bit for bit, and a
    changed KV length gets its own plan."""
    b = W.cascade_shared_prefix(seed=2008, groups=2, members=6, prefix_tokens=768,
                                suffix_max=200, extra=2, extra_tokens=300)
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=256,
                               l1_partition_tokens=256)
    cache = gpu.PlanCache(4)
    outs = []
    for layer in range(3):
        plan, hit = cache.get(b.indptr, b.indices, b.kv_len, b.page_size, params)
        assert hit == (layer > 0)
        o, l = plan.run(pool, q, b.sm_scale)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), l.cpu().numpy()))
    fo, fl, _ = cascade(gpu, b, params, pool, q)
    for o, l in outs:
        assert np.array_equal(o, fo) and np.array_equal(l, fl)
    kl = b.kv_len.copy()
    kl[0] -= 1
    plan, hit = cache.get(b.indptr, b.indices, kl, b.page_size, params)
    assert not hit


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_nested_sharing(gpu, depth):
    """A system prompt shared by every tenant's requests and a sub-prefix per
    tenant: one span level (the page's), or the tenant spans nested below it,
    all in the one level-0 launch; equal to the oracle and to the flat
    launch, and the same with both levels in one grid or two launches."""
    b = W.nested_shared_prefix(seed=2510, tenants=3, members=5, system_tokens=512,
                               tenant_tokens=256, suffix_max=300, extra=3, extra_tokens=600)
    pool, csr, q = to_device(b)
    res = {}
    for fuse in (1, 0):
        params = gpu.CascadeParams(enabled=1, max_groups=0, max_depth=depth, fuse_levels=fuse,
                                   l0_partition_tokens=256, l1_partition_tokens=256)
        out, lse, plan = cascade(gpu, b, params, pool, q)
        assert len(plan.field("span_pages")) == (1 if depth == 1 else 4)
        res[fuse] = (out, lse)
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    out, lse = res[1]
    ro, rl = oatt.decode_attention(b)
    assert_close(out, ro, TOL["bf16"], "nested cascade out")
    assert_lse(lse, rl, "nested cascade lse")
    fo, fl, _ = flat_decode(b, pool, csr, q, 256)
    assert rel_err(out, fo.cpu().numpy()) <= 1e-5
    assert lse_err(lse, fl.cpu().numpy()) <= 1e-5


def test_nested_full_workload_sampled(gpu):
    """The benchmark's nested workload at full size (batch 72, 2048-token
    system prompt, 4 tenant sub-prefixes of 2048 tokens) with nested spans:
    sampled requests against the oracle, all of it against the flat launch."""
    b = W.nested_shared_prefix()
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, max_groups=0, max_depth=2, l0_partition_tokens=1024,
                               l1_partition_tokens=512)
    out, lse, plan = cascade(gpu, b, params, pool, q)
    assert len(plan.field("span_pages")) == 5
    fo, fl, _ = flat_decode(b, pool, csr, q, 512)
    assert rel_err(out, fo.cpu().numpy()) <= 1e-5
    assert lse_err(lse, fl.cpu().numpy()) <= 1e-5
    reqs = [0, 9, 40, 71]
    ro, rl = oatt.decode_attention(b, requests=reqs)
    assert_close(out[reqs], ro[reqs], TOL["bf16"], "nested out")
    assert_lse(lse[reqs], rl[reqs], "nested lse")


def test_declined_plan_runs_flat(gpu):
    b = W.llama3_8b_flat(seed=2005, batch=5, min_len=100, max_len=900)
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1)
    out, lse, plan = cascade(gpu, b, params, pool, q)
    assert plan.stats()[1] == "no_candidate"
    fo, fl, _ = flat_decode(b, pool, csr, q, 512)
    assert np.array_equal(out, fo.cpu().numpy()) and np.array_equal(lse, fl.cpu().numpy())


def test_cascade_full_workload_sampled(gpu):
    """Batch 72: 4 groups x 16 members sharing 4096-token prefixes plus 8
    non-members; all groups at level 0 (and the single-subgroup plan)."""
    b = W.cascade_shared_prefix()
    pool, csr, q = to_device(b)
    fo, fl, _ = flat_decode(b, pool, csr, q, 512)
    fo, fl = fo.cpu().numpy(), fl.cpu().numpy()
    reqs = [0, 5, 31, 70, 71]
    ro, rl = oatt.decode_attention(b, requests=reqs)
    assert_close(fo[reqs], ro[reqs], TOL["bf16"], "flat out")
    for mg in (0, 1):
        params = gpu.CascadeParams(enabled=1, max_groups=mg, l0_partition_tokens=256,
                                   l1_partition_tokens=512)
        out, lse, plan = cascade(gpu, b, params, pool, q)
        assert plan.stats()[0]["members"] == (64 if mg == 0 else 16)
        assert np.all(np.isfinite(out))
        assert rel_err(out, fo) <= 1e-5, mg
        assert lse_err(lse, fl) <= 1e-5, mg
        assert_close(out[reqs], ro[reqs], TOL["bf16"], "cascade out")
        assert_lse(lse[reqs], rl[reqs], "cascade lse")


def test_single_merge_equals_two_stage_form(gpu):
    """The page's form: level-0 states (stacked launch, merged), unstacked,
    level-1 states (merged), then the [level 0, level 1] pair merge."""
    b = W.tiny_gqa_fp32()
    pool, csr, q = to_device(b)
    params = gpu.CascadeParams(enabled=1, min_shared_pages=2, l0_partition_tokens=32,
                               l1_partition_tokens=32)
    fused, fused_lse, plan = cascade(gpu, b, params, pool, q)
    members = plan.field("members")
    M, Hkv, Hq, G = len(members), b.num_kv_heads, b.num_q_heads, b.group
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    q0 = gpu.stack_heads(q, dev(members), Hkv).reshape(1, M * Hq, -1).contiguous()
    l0 = gpu.DeviceCSR.from_host(plan.field("l0_indptr"), plan.field("l0_indices"),
                                 plan.field("l0_len"))
    p0 = gpu.partition_indptr(plan.field("l0_len"), 32)
    v0, s0 = gpu.paged_decode_partial(pool, l0, q0, b.sm_scale, 32, dev(p0), int(p0[-1]))
    m0, ml0 = gpu.merge_states(v0, s0, dev(p0))
    u0, ul0 = gpu.unstack_heads(m0[0].contiguous(), ml0[0].contiguous(), M, Hkv, G)
    l1 = gpu.DeviceCSR.from_host(plan.field("l1_indptr"), plan.field("l1_indices"),
                                 plan.field("l1_len"))
    p1 = gpu.partition_indptr(plan.field("l1_len"), 32)
    v1, s1 = gpu.paged_decode_partial(pool, l1, q, b.sm_scale, 32, dev(p1), int(p1[-1]))
    m1, ml1 = gpu.merge_states(v1, s1, dev(p1))
    mind = plan.field("merge_indptr")
    rows_v = torch.empty((int(mind[-1]), Hq, b.head_dim_v), device="cuda")
    rows_l = torch.empty((int(mind[-1]), Hq), device="cuda")
    rank = plan.field("member_rank")
    for r in range(b.batch):
        at = int(mind[r])
        if rank[r] >= 0:
            rows_v[at], rows_l[at] = u0[rank[r]], ul0[rank[r]]
            at += 1
        rows_v[at], rows_l[at] = m1[r], ml1[r]
    two, two_l = gpu.merge_states(rows_v, rows_l, dev(mind))
    assert rel_err(two.cpu().numpy(), fused) <= 1e-5
    assert lse_err(two_l.cpu().numpy(), fused_lse) <= 1e-5


def test_stack_unstack_match_the_head_map(gpu):
    rng = np.random.default_rng(9)
    B, Hkv, G, D = 7, 4, 3, 16
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, D)).astype(np.float32)).cuda()
    members = np.array([1, 4, 6], np.int32)
    q0 = gpu.stack_heads(q, torch.from_numpy(members).cuda(), Hkv).cpu().numpy()
    hmap = oplan.stacked_head_map(3, Hkv, G)
    qn = q.cpu().numpy()
    for h0, t in enumerate(hmap):
        m, i = divmod(int(t), Hkv * G)
        assert np.array_equal(q0[h0], qn[members[m], i])
    v0 = torch.from_numpy(rng.standard_normal((3 * Hkv * G, D)).astype(np.float32)).cuda()
    l0 = torch.from_numpy(rng.standard_normal(3 * Hkv * G).astype(np.float32)).cuda()
    v, l = gpu.unstack_heads(v0, l0, 3, Hkv, G)
    v, l, v0n, l0n = v.cpu().numpy(), l.cpu().numpy(), v0.cpu().numpy(), l0.cpu().numpy()
    for h0, t in enumerate(hmap):
        m, i = divmod(int(t), Hkv * G)
        assert np.array_equal(v[m, i], v0n[h0]) and l[m, i] == l0n[h0]


def test_member_major_stacking_reads_the_wrong_kv_head(gpu):
    """Negative control: the stacked level-0 launch fed member-major queries
    (h0 = m*Hq + kv*G + g) reads the wrong KV head and misses the oracle."""
    b = W.tiny_gqa_fp32()
    pool, csr, q = to_device(b)
    plan = oplan.build_cascade_plan(b.indptr, b.indices, b.kv_len, 16,
                                    oplan.CascadeParams(enabled=1, min_shared_pages=2))
    members = plan.members
    M, Hq = len(members), b.num_q_heads
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    good_q0 = gpu.stack_heads(q, dev(members), b.num_kv_heads).reshape(1, M * Hq, -1).contiguous()
    bad_q0 = q[torch.from_numpy(members.astype(np.int64)).cuda()].reshape(1, M * Hq, -1).contiguous()
    l0 = gpu.DeviceCSR.from_host(plan.l0_indptr, plan.l0_indices, plan.l0_len)
    p0 = gpu.partition_indptr(plan.l0_len, 32)
    res = {}
    for name, q0 in (("kv_major", good_q0), ("member_major", bad_q0)):
        v, s = gpu.paged_decode_partial(pool, l0, q0, b.sm_scale, 32, dev(p0), int(p0[-1]))
        o, _ = gpu.merge_states(v, s, dev(p0))
        res[name] = o[0].cpu().numpy()
    # reference: each member's own heads over the shared span, by definition
    qf = b.q.astype(np.float64)
    K, V = oatt.gather(b.k_pool, b.v_pool, "f32", 1.0, 1.0, plan.l0_indptr, plan.l0_indices,
                       plan.l0_len, 16, 0, 64)
    want = np.zeros((M, Hq, 64))
    for m in range(M):
        want[m], _ = oatt.attend(qf[members[m]], K, V, b.sm_scale, b.group)
    hmap = oplan.stacked_head_map(M, b.num_kv_heads, b.group)
    kv_major = np.stack([want[t // Hq, t % Hq] for t in hmap])
    member_major = want.reshape(M * Hq, 64)   # row m*Hq + i is member m's head i
    assert rel_err(res["kv_major"], kv_major) <= 1e-5
    assert rel_err(res["member_major"], member_major) > 1e-2


def test_plan_runs_repeat_and_cover_empty_requests(gpu):
    """Repeated runs of one uploaded plan agree bit for bit (no state is
    carried between runs), with and without sharing, and an empty request
    still gets (0, -inf)."""
    lens = [300, 0, 530, 530, 17, 0, 530]
    b = W.random_batch(81, batch=len(lens), page_size=16, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, kv_dtype="bf16", q_dtype="bf16", min_len=0, max_len=0,
                       partition_tokens=128, lens=lens, share=[([2, 3, 6], 20)])
    pool, csr, q = to_device(b)
    ro, rl = oatt.decode_attention(b)
    for enabled in (0, 1):
        plan = gpu.CascadePlan(b.indptr, b.indices, b.kv_len, 16,
                               gpu.CascadeParams(enabled=enabled, min_shared_pages=4,
                                                 l0_partition_tokens=64, l1_partition_tokens=128))
        outs = []
        for _ in range(3):
            o, l = plan.run(pool, q, b.sm_scale)
            torch.cuda.synchronize()
            outs.append((o.cpu().numpy(), l.cpu().numpy()))
        assert plan.stats()[0]["members"] == (3 if enabled else 0)
        for o, l in outs[1:]:
            assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
        o, l = outs[0]
        assert_close(o, ro, TOL["bf16"], "planned out")
        assert_lse(l, rl, "planned lse")
        assert np.all(o[[1, 5]] == 0) and np.all(l[[1, 5]] == -np.inf)
