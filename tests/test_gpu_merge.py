"""merge_states on the GPU against the oracle merge [cascade-PR, "How the
#898 merge kernel is reused"]: parity, the bit-exact identity of one-row
groups, -inf rows and empty groups, associativity across regroupings, the
natural-log negative control, and the full 8192 x 32 x 128 workload on
sampled rows."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from workloads import merge_microbench
from gpu_util import assert_close, assert_lse, lse_err, rel_err

pytestmark = pytest.mark.gpu


def run_merge(pdk, v, l, ind):
    vt = torch.from_numpy(v).cuda()
    lt = torch.from_numpy(l).cuda()
    it = torch.from_numpy(ind.astype(np.int32)).cuda()
    vo, lo = pdk.merge_states(vt, lt, it)
    torch.cuda.synchronize()
    return vo.cpu().numpy(), lo.cpu().numpy()


def test_merge_small_matches_oracle(gpu):
    m = merge_microbench(seed=7, M=300, H=4, D=128)
    vo, lo = run_merge(gpu, m.v_in, m.lse_in, m.o_indptr)
    ro, rl = oatt.merge_states(m.v_in, m.lse_in, m.o_indptr)
    assert_close(vo, ro, 1e-5, "merge out")
    assert_lse(lo, rl, "merge lse")


def test_merge_ragged_width_and_tail(gpu):
    # H*D = 3*68 is not a multiple of the 1024-float workgroup span
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 7, size=50)
    ind = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    v = rng.standard_normal((ind[-1], 3, 68)).astype(np.float32)
    l = rng.uniform(-4, 20, (ind[-1], 3)).astype(np.float32)
    l[rng.random(l.shape) < 0.2] = -np.inf
    v[np.isinf(l)] = np.nan  # rows with lse = -inf must not be read into the sum
    vo, lo = run_merge(gpu, v, l, ind)
    ro, rl = oatt.merge_states(np.where(np.isnan(v), 0, v), l, ind)
    assert np.all(np.isfinite(vo))
    assert_close(vo, ro, 1e-5, "merge out")
    assert_lse(lo, rl, "merge lse")
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 0
    assert np.all(vo[empty] == 0) and np.all(lo[empty] == -np.inf)


def test_merge_group_of_one_is_bit_exact(gpu):
    rng = np.random.default_rng(4)
    v = rng.standard_normal((257, 8, 64)).astype(np.float32)
    l = rng.uniform(-30, 30, (257, 8)).astype(np.float32)
    vo, lo = run_merge(gpu, v, l, np.arange(258, dtype=np.int32))
    assert np.array_equal(vo.view(np.uint32), v.view(np.uint32))
    assert np.array_equal(lo.view(np.uint32), l.view(np.uint32))


def test_merge_is_associative_across_regroupings(gpu):
    rng = np.random.default_rng(5)
    counts = rng.integers(1, 12, size=200)
    ind = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    v = rng.standard_normal((ind[-1], 4, 32)).astype(np.float32)
    l = rng.uniform(-4, 20, (ind[-1], 4)).astype(np.float32)
    one_o, one_l = run_merge(gpu, v, l, ind)
    sub, outer = [0], [0]
    for j in range(len(counts)):
        a, e = ind[j], ind[j + 1]
        cuts = sorted(set(rng.integers(a + 1, e + 1, size=rng.integers(0, 4)).tolist()) | {e})
        sub += cuts
        outer.append(len(sub) - 1)
    so, sl = run_merge(gpu, v, l, np.array(sub, np.int32))
    two_o, two_l = run_merge(gpu, so, sl, np.array(outer, np.int32))
    assert rel_err(two_o, one_o) <= 1e-5
    assert lse_err(two_l, one_l) <= 1e-5


def test_natural_log_lse_is_rejected_by_the_log2_merge(gpu):
    """Negative control: natural-log LSEs through the log2 merge miss the
    oracle by far more than the tolerance."""
    rng = np.random.default_rng(8)
    ind = np.arange(0, 257, 4, dtype=np.int32)          # 64 groups of 4 rows
    v = rng.standard_normal((256, 4, 64)).astype(np.float32)
    l = rng.uniform(-4, 20, (256, 4)).astype(np.float32)  # spread well over 4 units
    ro, _ = oatt.merge_states(v, l, ind)
    good, _ = run_merge(gpu, v, l, ind)
    bad, _ = run_merge(gpu, v, (l * math.log(2.0)).astype(np.float32), ind)
    assert rel_err(good, ro) <= 1e-5
    assert rel_err(bad, ro) > 100 * 1e-5


def test_merge_full_workload_sampled(gpu):
    """8192 output rows, H 32, D 128, counts uniform in 1..16 (the launch the
    benchmark times), checked on sampled rows plus every one-row group."""
    m = merge_microbench()
    vo, lo = run_merge(gpu, m.v_in, m.lse_in, m.o_indptr)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(len(m.o_indptr) - 1, size=256, replace=False))
    for i in rows:
        a, e = m.o_indptr[i], m.o_indptr[i + 1]
        ro, rl = oatt.merge_states(m.v_in[a:e], m.lse_in[a:e], np.array([0, e - a]))
        assert_close(vo[i:i + 1], ro, 1e-5, f"row {i}")
        assert_lse(lo[i:i + 1], rl, f"row {i}")
    ones = np.nonzero(np.diff(m.o_indptr) == 1)[0]
    assert len(ones) > 100
    src = m.o_indptr[ones]
    assert np.array_equal(vo[ones].view(np.uint32), m.v_in[src].view(np.uint32))
    assert np.array_equal(lo[ones].view(np.uint32), m.lse_in[src].view(np.uint32))


def test_merge_groups_longer_than_one_round_trip(gpu):
    """Groups of more than 16 rows are folded batch by batch: an all-empty
    first batch (skipped), a maximum that first appears in a later batch
    (running rescale), lengths on and past the batch boundaries."""
    rng = np.random.default_rng(9)
    counts = np.array([17, 32, 33, 40, 16, 1, 0, 48, 21, 64], dtype=np.int64)
    ind = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    H, D = 4, 64
    v = rng.standard_normal((ind[-1], H, D)).astype(np.float32)
    l = rng.uniform(-4, 20, (ind[-1], H)).astype(np.float32)
    a = ind[8]                       # group of 21: rows 0..15 empty
    l[a:a + 16] = -np.inf
    v[a:a + 16] = np.nan             # never read into the sum
    b = ind[9]                       # group of 64: the largest LSEs in the last batch
    l[b:b + 48] = rng.uniform(-30, -20, (48, H)).astype(np.float32)
    l[b + 48:b + 64] = rng.uniform(25, 30, (16, H)).astype(np.float32)
    vo, lo = run_merge(gpu, v, l, ind)
    ro, rl = oatt.merge_states(np.where(np.isnan(v), 0, v), l, ind)
    assert np.all(np.isfinite(vo))
    assert_close(vo, ro, 1e-5, "merge out")
    assert_lse(lo, rl, "merge lse")
