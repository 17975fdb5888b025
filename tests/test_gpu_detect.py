"""Shared-prefix detection on the device (page ids only on the GPU)
[cascade-PR, "Detection reads the page table, not the refcounts"]: every
plan field, the stats and the decline reason equal the oracle planner's
(oracle/planner.py, and oracle/nested.py for nested spans) and the host
planner's for the same table; decode outputs of the device plan (its views'
page ids gathered on the device at upload) are bit-identical to the host
plan's and within the bf16 bar of the oracle's attention;
tables with thousands of requests (the grouping scan crosses many
64-request chunks) and every rejection case; misuse is refused."""
import numpy as np
import pytest
import torch

import paged_split_kv_v2_amd as pdk
import workloads as W
from gpu_util import TOL, assert_close, assert_lse, to_device
from oracle import attention as oatt
from plan_expect import expected_plan

pytestmark = pytest.mark.gpu

FIELDS = ("members", "group_indptr", "span_pages", "span_start", "span_parent", "l0_indptr",
          "l0_len", "l1_indptr", "l1_len", "merge_indptr", "fused_merge_indptr", "group_of",
          "member_rank")


def both(gpu, indptr, indices, kv_len, P, **kw):
    """The device-detected plan against the oracle's plan and the host
    plan, field by field; returns (host plan, device plan)."""
    params = gpu.CascadeParams(**kw)
    host = gpu.CascadePlan(indptr, indices, kv_len, P, params)
    csr = gpu.DeviceCSR.from_host(indptr, indices, kv_len)
    dev = gpu.CascadePlan.from_device(csr, indptr, kv_len, P, params)
    want, stats, decline = expected_plan(indptr, indices, kv_len, P, kw)
    for f in FIELDS:
        assert np.array_equal(dev.field(f).astype(np.int64),
                              np.asarray(want[f], np.int64)), f
        assert np.array_equal(host.field(f), dev.field(f)), f
    got_stats, got_decline = dev.stats()
    assert got_decline == decline
    if stats is not None:
        assert got_stats == stats
    assert host.stats() == dev.stats()
    assert dev.field("l0_indices").size == 0 and dev.field("l1_indices").size == 0
    return host, dev


def random_shared_table(rng, B, groups, P=16):
    lists, nxt = [], 0
    heads = []
    for g in range(groups):
        n = int(rng.integers(1, 12))
        heads.append(list(range(nxt, nxt + n)))
        nxt += n
    for b in range(B):
        pl = []
        if rng.random() < 0.9:
            h = heads[int(rng.integers(0, groups))]
            pl = h[:int(rng.integers(1, len(h) + 1))]     # early divergence shortens spans
        k = int(rng.integers(0, 6))
        pl = pl + list(range(nxt, nxt + k))
        nxt += k
        lists.append(pl)
    kv = [max(0, len(pl) * P - int(rng.integers(0, P))) if pl else 0 for pl in lists]
    indptr = np.cumsum([0] + [len(pl) for pl in lists]).astype(np.int32)
    indices = np.asarray([p for pl in lists for p in pl] or [0], np.int32)[:indptr[-1]]
    return indptr, indices, np.asarray(kv, np.int32)


@pytest.mark.parametrize("max_groups", [0, 1, 3])
def test_device_plan_equals_host_plan_on_random_tables(gpu, max_groups):
    rng = np.random.default_rng(2600 + max_groups)
    for B, groups in ((7, 2), (130, 5), (3000, 40)):
        ip, ix, kl = random_shared_table(rng, B, groups)
        for mp, mm in ((1, 2), (4, 3), (2, 20)):
            both(gpu, ip, ix, kl, 16, enabled=1, max_groups=max_groups, min_shared_pages=mp,
                 min_members=mm, l0_partition_tokens=64, l1_partition_tokens=128)


def test_declines_match(gpu):
    b = W.llama3_8b_flat(seed=2610, batch=9, min_len=10, max_len=900, poison=False)
    for enabled in (0, 1):
        _, dev = both(gpu, b.indptr, b.indices, b.kv_len, 16, enabled=enabled)
        assert dev.stats()[1] == ("disabled" if enabled == 0 else "no_candidate")


def test_device_plan_runs_bit_identical(gpu):
    b = W.cascade_shared_prefix(seed=2620, groups=3, members=6, prefix_tokens=1024,
                                suffix_max=300, extra=3, extra_tokens=700)
    pool, csr, q = to_device(b)
    host, dev = both(gpu, b.indptr, b.indices, b.kv_len, b.page_size, enabled=1, max_groups=0,
                     l0_partition_tokens=256, l1_partition_tokens=512)
    ho, hl = host.run(pool, q, b.sm_scale)
    do, dl = dev.run(pool, q, b.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(ho, do) and torch.equal(hl, dl)
    ro, rl = oatt.decode_attention(b)
    assert_close(do.cpu().numpy(), ro, TOL["bf16"], "device-planned cascade out")
    assert_lse(dl.cpu().numpy(), rl, "device-planned cascade lse")


def test_misuse_is_refused(gpu):
    b = W.cascade_shared_prefix(seed=2630, groups=2, members=4, prefix_tokens=512,
                                suffix_max=200, extra=1, extra_tokens=300)
    csr = gpu.DeviceCSR.from_host(b.indptr, b.indices, b.kv_len)
    bad = b.kv_len.copy()
    bad[0] += 64                          # 4 more pages than the table holds
    with pytest.raises(gpu.PdkError):
        gpu.CascadePlan.from_device(csr, b.indptr, bad, 16, gpu.CascadeParams(enabled=1))
    dev = gpu.CascadePlan.from_device(csr, b.indptr, b.kv_len, 16,
                                      gpu.CascadeParams(enabled=1, max_groups=0))
    ws = torch.empty(dev.workspace_bytes(32, 128), dtype=torch.uint8, device="cuda")
    # the plain upload would leave the views' page ids unset
    assert gpu.lib().pdk_cascade_plan_upload(dev._h, ws.data_ptr(), ws.numel(), None) != 0


def random_nested_table(rng, B, P=16):
    """Requests walking down a random forest of shared page runs (root run,
    then one of its child runs, then a grandchild run), then private pages."""
    nxt = 0
    def run(n):
        nonlocal nxt
        r = list(range(nxt, nxt + n))
        nxt += n
        return r
    roots = [run(int(rng.integers(1, 5))) for _ in range(3)]
    kids = [[run(int(rng.integers(1, 4))) for _ in range(int(rng.integers(1, 4)))]
            for _ in roots]
    grand = [[[run(int(rng.integers(1, 3))) for _ in range(2)] for _ in k] for k in kids]
    lists = []
    for _ in range(B):
        i = int(rng.integers(0, len(roots)))
        pl = list(roots[i])
        if rng.random() < 0.85:
            j = int(rng.integers(0, len(kids[i])))
            pl += kids[i][j]
            if rng.random() < 0.7:
                pl += grand[i][j][int(rng.integers(0, 2))]
        pl += run(int(rng.integers(0, 4)))
        lists.append(pl)
    kv = [len(pl) * P - int(rng.integers(0, P)) for pl in lists]
    indptr = np.cumsum([0] + [len(pl) for pl in lists]).astype(np.int32)
    indices = np.asarray([p for pl in lists for p in pl], np.int32)
    return indptr, indices, np.asarray(kv, np.int32)


@pytest.mark.parametrize("max_depth", [2, 3, 4])
def test_device_nested_plans_equal_host_plans(gpu, max_depth):
    rng = np.random.default_rng(2640 + max_depth)
    deep = 0
    for B in (6, 40, 300):
        for _ in range(6):
            ip, ix, kl = random_nested_table(rng, B)
            host, _ = both(gpu, ip, ix, kl, 16, enabled=1, max_groups=0, min_shared_pages=1,
                           max_depth=max_depth, l0_partition_tokens=64,
                           l1_partition_tokens=128)
            deep += int((host.field("span_parent") >= 0).sum())
    assert deep > 0    # the tables do produce nested spans


def test_device_nested_plan_runs_bit_identical(gpu):
    b = W.nested_shared_prefix(seed=2650, tenants=3, members=5, system_tokens=512,
                               tenant_tokens=256, suffix_min=1, suffix_max=200, extra=2,
                               extra_tokens=300)
    pool, csr, q = to_device(b)
    host, dev = both(gpu, b.indptr, b.indices, b.kv_len, b.page_size, enabled=1, max_groups=0,
                     max_depth=2, l0_partition_tokens=256, l1_partition_tokens=256)
    assert len(host.field("span_pages")) == 4     # system prompt + 3 tenant spans
    ho, hl = host.run(pool, q, b.sm_scale)
    do, dl = dev.run(pool, q, b.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(ho, do) and torch.equal(hl, dl)
