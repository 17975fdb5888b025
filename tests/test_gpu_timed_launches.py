"""Full-size parity of exactly the launches bench.py times, with the arm
parameters imported from bench.py: the Llama-3-8B-shaped flat step (a
declined plan's flat launch, longest partition first, 512-token
partitions) and the no-sharing gate's plan; every shared-prefix arm on the
batch-72 workload (flat, single subgroup, all groups in one grid at level-0
partitions of 1,024 tokens, all groups as two launches) and every pair of
partition sizes the autotuner may pick; every nested-sharing arm. Each run
is checked on sampled requests against the f64 oracle (bf16 KV: 2e-3, LSE
1e-4 log2 units) and as a whole against the GPU flat launch (1e-5)."""
import numpy as np
import pytest
import torch

import bench
import workloads as W
from oracle import attention as oatt
from gpu_util import TOL, assert_close, assert_lse, flat_decode, lse_err, rel_err, to_device

pytestmark = pytest.mark.gpu


def run_arm(gpu, b, pool, q, kw):
    plan = gpu.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, gpu.CascadeParams(**kw))
    out, lse = plan.run(pool, q, b.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), plan


def check(b, got, flat, ref, reqs, what):
    out, lse, _ = got
    fo, fl = flat
    ro, rl = ref
    assert np.all(np.isfinite(out)), what
    assert rel_err(out, fo) <= 1e-5 and lse_err(lse, fl) <= 1e-5, what
    assert_close(out[reqs], ro[reqs], TOL[b.kv_dtype], f"{what} out")
    assert_lse(lse[reqs], rl[reqs], f"{what} lse")


def reference(b, pool, csr, q, reqs, S=512):
    fo, fl, _ = flat_decode(b, pool, csr, q, S)
    return (fo.cpu().numpy(), fl.cpu().numpy()), oatt.decode_attention(b, requests=reqs)


def test_flat_and_gate_arms(gpu):
    b = W.llama3_8b_flat()
    pool, csr, q = to_device(b)
    reqs = [0, 13, 31, 47, 63]
    flat, ref = reference(b, pool, csr, q, reqs)
    got = run_arm(gpu, b, pool, q, bench.FLAT_ARM)
    assert got[2].stats()[1] == "disabled"
    check(b, got, flat, ref, reqs, "flat arm")
    gate = run_arm(gpu, b, pool, q, bench.GATE_ARM)
    assert gate[2].stats()[1] == "no_candidate"
    # the declined plan runs the same flat launch
    assert np.array_equal(gate[0], got[0]) and np.array_equal(gate[1], got[1])


def test_cascade_arms(gpu):
    b = W.cascade_shared_prefix()
    pool, csr, q = to_device(b)
    reqs = [0, 5, 31, 44, 70, 71]
    flat, ref = reference(b, pool, csr, q, reqs)
    members = {"flat": 0, "cascade_single_group": 16, "cascade_all_groups": 64,
               "cascade_all_groups_two_launches": 64}
    for name, kw in bench.CASCADE_ARMS:
        got = run_arm(gpu, b, pool, q, kw)
        assert got[2].stats()[0]["members"] == members[name], name
        check(b, got, flat, ref, reqs, name)


def test_autotuner_candidates(gpu):
    """Every (level-0, level-1) pair the benchmark's autotuned arm may pick."""
    b = W.cascade_shared_prefix()
    pool, csr, q = to_device(b)
    reqs = [3, 40, 66, 71]
    flat, ref = reference(b, pool, csr, q, reqs)
    for s0 in (256, 512, 1024, 2048):
        for s1 in (256, 512, 1024):
            got = run_arm(gpu, b, pool, q, dict(bench.CASCADE_TUNE_BASE,
                                                l0_partition_tokens=s0, l1_partition_tokens=s1))
            check(b, got, flat, ref, reqs, f"l0 {s0} / l1 {s1}")


def test_nested_arms(gpu):
    b = W.nested_shared_prefix()
    pool, csr, q = to_device(b)
    reqs = [0, 9, 40, 71]
    flat, ref = reference(b, pool, csr, q, reqs)
    spans = {"flat": 0, "one_span_level": 1, "nested_spans": 5}
    for name, kw in bench.NESTED_ARMS:
        got = run_arm(gpu, b, pool, q, kw)
        assert len(got[2].field("span_pages")) == spans[name], name
        check(b, got, flat, ref, reqs, name)
