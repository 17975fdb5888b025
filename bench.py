"""Benchmark: paged split-KV decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R]
                    [--workload flat|cascade|merge|mla|flat_mt|mla_mt|nested|copy]

A step is one attention layer's decode for the whole batch: every partial
launch and every merge of the path. Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts; plans (page-table
bookkeeping on the host) are built and uploaded before it, as they are
reused across a model's layers. Prints one JSON line.

Protocol: W untimed warmup steps, then R timed regions of exactly K steps
each, synchronized on both sides; ``ms_per_step`` and ``value`` come from
the median region and ``reps`` gives median / min / max. The default line
(``--workload flat``) measures its sub-workloads first (merge_states, the
MLA share, the shared-prefix arms, the no-sharing gate) and the headline
Llama-3-8B-shaped flat step last; the CPU oracle baseline runs before any
GPU work, on every host core it may use.

``value`` is the achieved rate over the batch's unique KV bytes (each
distinct page row read once) per step. ``roofline`` reports the dominant
kernel with its duration measured by HIP events on the stream it is
launched on (one event pair around back-to-back launches of that kernel,
median over the regions). Cold-cache figures time one step at a time after
a 512 MiB read that evicts the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attn: KV HBM GB/s (frac of peak) + µs/step; cascade vs flat"

# Launch parameters of every timed arm (pdk.CascadeParams keywords). The
# full-size parity tests (tests/test_gpu_timed_launches.py) run these same
# arms against the oracle.
FLAT_ARM = dict(enabled=0, l1_partition_tokens=512)
# cascade on with the default thresholds: on the no-sharing workload the
# detection scan declines and the flat launch runs
GATE_ARM = dict(enabled=1, l1_partition_tokens=512)
CASCADE_ARMS = (
    ("flat", dict(enabled=0, l1_partition_tokens=512)),
    ("cascade_single_group", dict(enabled=1, max_groups=1, l0_partition_tokens=512,
                                  l1_partition_tokens=512)),
    ("cascade_all_groups", dict(enabled=1, max_groups=0, l0_partition_tokens=1024,
                                l1_partition_tokens=512)),
    ("cascade_all_groups_two_launches", dict(enabled=1, max_groups=0, l0_partition_tokens=256,
                                             l1_partition_tokens=512, fuse_levels=0)),
)
CASCADE_TUNE_BASE = dict(enabled=1, max_groups=0)
NESTED_ARMS = (
    ("flat", dict(enabled=0, l1_partition_tokens=512)),
    ("one_span_level", dict(enabled=1, max_groups=0, max_depth=1, l0_partition_tokens=1024,
                            l1_partition_tokens=512)),
    ("nested_spans", dict(enabled=1, max_groups=0, max_depth=2, l0_partition_tokens=1024,
                          l1_partition_tokens=512)),
)
NESTED_TUNE_BASE = dict(enabled=1, max_groups=0, max_depth=2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats_of(values, nd=2):
    v = sorted(values)
    return {"median": round(statistics.median(v), nd), "min": round(v[0], nd),
            "max": round(v[-1], nd), "n": len(v)}


# --------------------------------------------------------------------------
# CPU baseline: the f64 oracle, as it stands, over the host cores
# --------------------------------------------------------------------------

_CPU_JOB = None


def cpu_workers() -> int:
    """Worker processes for the oracle: the cores this process may run on,
    capped by OMP_NUM_THREADS when it is set (the host's CPU share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(w):
    """Worker w runs units w, w + W, w + 2W, ... (cycling) for min_s seconds
    with one BLAS thread; returns (units done, summed amount, seconds)."""
    import threadpoolctl
    run, amount, order, workers, min_s = _CPU_JOB
    done, total = 0, 0.0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        i = w
        while time.perf_counter() - t0 < min_s:
            u = order[i % len(order)]
            run(u)
            done += 1
            total += amount(u)
            i += workers
    return done, total, time.perf_counter() - t0


def oracle_rate(units, run, amount, unit, scale, what, min_s=10.0):
    """The f64 oracle timed over a bounded sample of the workload on every
    host core it may use: one forked worker per core (before any GPU use),
    each running units in a seeded order for about min_s seconds; value =
    the summed amount per second of the slowest worker / scale."""
    import multiprocessing as mp
    global _CPU_JOB
    workers = cpu_workers()
    order = [units[i] for i in np.random.default_rng(0).permutation(len(units))]
    _CPU_JOB = (run, amount, order, workers, min_s)
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_cpu_worker, range(workers))
    _CPU_JOB = None
    done = sum(r[0] for r in res)
    total = sum(r[1] for r in res)
    dt = max(r[2] for r in res)
    return {"value": round(total / dt / scale, 4), "unit": unit, "cores": workers,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} {what} ({done / len(units):.2f} passes over the workload's "
                      f"{len(units)}), f64 numpy oracle, {workers} worker processes x 1 thread, "
                      f"{dt:.1f} s"}


def cpu_baseline_for(workload, x):
    """The oracle timed on the workload the GPU line measures (x: its host
    inputs), in the line's unit."""
    from oracle import attention as oatt
    if workload == "flat":
        return oracle_rate(list(range(x.batch)),
                           lambda r: oatt.decode_attention(x, requests=[r]),
                           lambda r: int(x.kv_len[r]) * x.kv_bytes_per_token(), "GB/s", 1e9,
                           "requests (all heads)")
    if workload in ("cascade", "nested"):
        from oracle import cascade as ocas, nested as onest, planner as opl
        p = opl.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=1024,
                              l1_partition_tokens=512)
        run = ((lambda _: ocas.cascade_decode(x, p)) if workload == "cascade"
               else (lambda _: onest.nested_cascade_decode(x, p, 2)))
        return oracle_rate([0], run, lambda _: x.unique_kv_bytes(), "GB/s", 1e9,
                           f"whole-batch {workload} decodes")
    if workload == "merge":
        ind, H, D = x.o_indptr, x.v_in.shape[1], x.v_in.shape[2]
        M = len(ind) - 1
        def run(u):
            a, e = int(ind[u]), int(ind[min(u + 64, M)])
            oatt.merge_states(x.v_in[a:e], x.lse_in[a:e], ind[u:min(u + 64, M) + 1] - a)
        def amount(u):
            rows = int(ind[min(u + 64, M)] - ind[u]) + min(64, M - u)
            return rows * H * (D + 1) * 4
        return oracle_rate(list(range(0, M, 64)), run, amount, "GB/s", 1e9,
                           "blocks of 64 output rows")
    if workload == "flat_mt":
        from oracle import multitoken as omt
        return oracle_rate(list(range(x.batch)),
                           lambda r: omt.multi_token_attention(x, True, requests=[r]),
                           lambda r: int(x.kv_len[r]) * x.kv_bytes_per_token(), "GB/s", 1e9,
                           "requests (all tokens and heads)")
    if workload in ("mla", "mla_mt"):
        from oracle import mla as omla, multitoken as omt
        pre, suf = x.prefix, x.suffix
        T = x.prefix.q.shape[1] if workload == "mla_mt" else 1
        flop_tok = 2 * pre.num_q_heads * (pre.head_dim_k + pre.head_dim_v)
        def amount(r):
            n = int(suf.kv_len[r])
            return flop_tok * (T * int(pre.kv_len[r]) + T * n - T * (T - 1) // 2)
        run = ((lambda r: omla.mla_flat(x, requests=[r])) if workload == "mla"
               else (lambda r: omt.mla_multi_token_flat(x, requests=[r])))
        return oracle_rate(list(range(pre.batch)), run, amount, "TFLOP/s", 1e12,
                           "requests (all heads)")
    return None


# --------------------------------------------------------------------------
# Device helpers and timing
# --------------------------------------------------------------------------

def dev_tensor(torch, a, device):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_batch(torch, pdk, b, device):
    pool = pdk.KVPool(k=dev_tensor(torch, b.k_pool, device),
                      v=None if b.v_pool is None else dev_tensor(torch, b.v_pool, device),
                      head_dim_v=b.head_dim_v, k_scale=b.k_scale, v_scale=b.v_scale)
    csr = pdk.DeviceCSR.from_host(b.indptr, b.indices, b.kv_len, device)
    return pool, csr, dev_tensor(torch, b.q, device)


class Timer:
    """HIP events on the current stream: every launch of the path is
    enqueued on the current (torch) stream, so an event pair brackets exactly
    the launches issued between its two records."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)
        return len(self.marks) - 1

    def us(self, a, b):
        return 1000.0 * self.marks[a].elapsed_time(self.marks[b])


def time_steps(torch, parts, steps, warmup, reps):
    """`warmup` untimed steps, then `reps` regions of exactly `steps` steps,
    each synchronized on both sides, each step running the callables in
    `parts` in order with nothing else enqueued between them. Then, for each
    part, its device time per call from `reps` event-bracketed runs of
    `steps` back-to-back calls of that part alone (time_launches). Returns
    (wall ms per step of each region, [per-part list of us per call])."""
    for _ in range(warmup):
        for f in parts:
            f()
    torch.cuda.synchronize()
    region_ms = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for f in parts:
                f()
        torch.cuda.synchronize()
        region_ms.append((time.perf_counter() - t0) * 1000.0 / steps)
    return region_ms, [[time_launches(torch, f, steps) for _ in range(reps)] for f in parts]


def time_launches(torch, f, n):
    """Device time (us) of one call of f: one HIP event pair on the current
    stream around n back-to-back calls (no event between two calls, since
    each one adds microseconds to a short launch). The span includes the
    gaps between the launches, so this is an upper bound on the kernel's own
    duration."""
    f()
    timer = Timer(torch)
    a = timer.mark()
    for _ in range(n):
        f()
    b = timer.mark()
    torch.cuda.synchronize()
    return timer.us(a, b) / n


def time_cold(torch, parts, steps, dev):
    """Device time (us) of each of `steps` steps, each run after a 512 MiB
    device read (a sum) that evicts the step's data from the 256 MB
    last-level (MALL) cache, as the other layers of a model would between
    two decode steps of one layer. The read is outside the timed span; HIP
    events bracket the step's launches. A read, not a write: evicting dirty
    lines would charge their write-back to the step."""
    scratch = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    for _ in range(2):
        scratch.sum()
    timer = Timer(torch)
    spans = []
    for _ in range(steps):
        scratch.sum()
        a = timer.mark()
        for f in parts:
            f()
        spans.append((a, timer.mark()))
    torch.cuda.synchronize()
    del scratch
    return [timer.us(a, b) for a, b in spans]


def kernel_source_files(kernel_source):
    """The kernel's translation unit and every local header it includes,
    directly or through other local headers, in first-include order."""
    import re
    csrc = os.path.join(ROOT, "paged_split_kv_v2_amd", "csrc")
    order, todo = [], [kernel_source]
    while todo:
        name = todo.pop(0)
        path = os.path.join(csrc, name)
        if name in order or not os.path.exists(path):
            continue
        order.append(name)
        todo += re.findall(r'^#include "([^"]+)"', open(path).read(), re.M)
    return order


def kernel_source_sha(kernel_source):
    """sha256 over the kernel's translation unit and the local headers it
    includes (kernel_source_files order)."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_split_kv_v2_amd", "csrc")
    if not os.path.exists(os.path.join(csrc, kernel_source)):
        return None
    h = hashlib.sha256()
    for name in kernel_source_files(kernel_source):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def counter_record(kernel_source, workload=None):
    """The committed rocprofv3 counter record of a kernel (profiles/
    counters.json, under its source file name, or "<source>|<workload>" for
    a second workload of one kernel), or None when the kernel's sources have
    changed since the counters were taken."""
    rec_path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(rec_path):
        return None
    key = kernel_source if workload is None else f"{kernel_source}|{workload}"
    rec = json.load(open(rec_path)).get(key)
    sha = kernel_source_sha(kernel_source)
    if not rec or sha is None or rec.get("source_sha256") != sha:
        return None
    return rec


def traffic_record(kernel_source, workload=None):
    """HBM bytes per launch from the kernel's counter record (FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by what the counter reads for a
    plain copy of known size), or None."""
    rec = counter_record(kernel_source, workload)
    if not rec or "fetch_kib_per_dispatch" not in rec:
        return None
    return int(rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_factor"] +
               rec["write_kib_per_dispatch"] * 1024 * rec["write_factor"])


def mfma_busy_record(kernel_source, workload=None):
    """Matrix-core busy fraction of the kernel from its counter record, or None."""
    rec = counter_record(kernel_source, workload)
    return None if not rec else rec.get("mfma_busy")


def params_of(pdk, kw):
    return pdk.CascadeParams(**kw)


def planned(torch, pdk, b, params, dev):
    """The plan, uploaded, and the host time of building it (us)."""
    plan = pdk.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, params)
    t0 = time.perf_counter()
    plan2 = pdk.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, params)
    plan_us = (time.perf_counter() - t0) * 1e6
    del plan2
    plan.upload(b.num_q_heads, b.head_dim_v, dev)
    return plan, plan_us


def plan_cache_hit_us(pdk, b, params, reps=200):
    """Host time of a plan-cache lookup that hits (the key compared): what
    every layer after the first pays for its plan."""
    cache = pdk.PlanCache(2)
    cache.get(b.indptr, b.indices, b.kv_len, b.page_size, params)
    t0 = time.perf_counter()
    for _ in range(reps):
        cache.get(b.indptr, b.indices, b.kv_len, b.page_size, params)
    return (time.perf_counter() - t0) * 1e6 / reps


def plan_parts(torch, b, pool, q, plan, dev):
    out = torch.empty((b.batch, b.num_q_heads, b.head_dim_v), dtype=torch.float32, device=dev)
    lse = torch.empty((b.batch, b.num_q_heads), dtype=torch.float32, device=dev)
    return [lambda: plan.run_partials(pool, q, b.sm_scale), lambda: plan.run_merge(out, lse)]


def run_plan_steps(args, torch, b, pool, q, plan, dev):
    """Timed steps of a planned decode: (region ms per step, partials us per
    region, merge us per region, cold-cache us per step)."""
    parts = plan_parts(torch, b, pool, q, plan, dev)
    region_ms, (t_part, t_merge) = time_steps(torch, parts, args.steps, args.warmup, args.reps)
    cold_us = time_cold(torch, parts, max(args.steps, 10), dev)
    return region_ms, t_part, t_merge, cold_us


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

def flat_line(args, torch, pdk, b, pool, q, plan, plan_us, dev):
    """The Llama-3-8B-shaped flat step (the headline): a declined plan's
    flat launch (longest partition first) and the merge."""
    S = FLAT_ARM["l1_partition_tokens"]
    region_ms, t_part, t_merge, cold_us = run_plan_steps(args, torch, b, pool, q, plan, dev)
    stats, _ = plan.stats()
    R = stats["suffix_chunks"]
    Hq, Dv = b.num_q_heads, b.head_dim_v
    kv = b.unique_kv_bytes()
    # the dominant kernel (partials): every KV byte once, the queries, the
    # page table, and the partial states it writes
    alg = (kv + b.q.nbytes + R * Hq * (Dv + 1) * 4 + b.indices.nbytes + b.kv_len.nbytes
           + (b.batch + 1) * 4)
    ms = statistics.median(region_ms)
    part_us = statistics.median(t_part)
    value = kv / (ms * 1e-3) / 1e9
    achieved = alg / (part_us * 1e-6) / 1e9
    cold = stats_of(cold_us)
    return {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_flat_paged_decode", "batch": b.batch,
                   "num_q_heads": Hq, "num_kv_heads": b.num_kv_heads, "head_dim": Dv,
                   "page_size": b.page_size, "partition_tokens": S,
                   "context_tokens": "uniform[1024,8192]", "total_tokens": int(b.kv_len.sum()),
                   "partitions": R, "kv_dtype": "bf16", "query_dtype": "bf16",
                   "parallelism": "none (1 GPU)"},
        "us_per_step": round(ms * 1000, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "reps": {"regions_of_steps": args.reps,
                 "us_per_step": stats_of([m * 1000 for m in region_ms])},
        "unique_kv_bytes": kv,
        "plan_host_us": round(plan_us, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record("partial_valu.hip"),
                     "kernel": "partial_valu_kernel<bf16,bf16,D128,4 rows>",
                     "kernel_us": round(part_us, 2), "kernel_us_reps": stats_of(t_part),
                     "bytes_per_launch": alg},
        "kernels_us": {"partials": stats_of(t_part), "merge": stats_of(t_merge)},
        "cold_cache": {"us_per_step": cold,
                       "unique_kv_GBps": round(kv / (cold["median"] * 1e-6) / 1e9, 2)},
    }


def gate_arm(args, torch, pdk, b, pool, q, flat_plan, dev):
    """The no-sharing overhead gate [cascade-PR, "How to run the
    benchmarks"]: the flat workload's shapes with nothing shared, the flat
    launch alone against the same launch behind the shared-prefix detection
    scan of every step (cascade on, default thresholds: the plan declines),
    and behind a plan-cache lookup (what each layer after the first pays)."""
    parts = plan_parts(torch, b, pool, q, flat_plan, dev)
    gate_params = params_of(pdk, GATE_ARM)
    probe = pdk.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, gate_params)
    _, decline = probe.stats()
    del probe

    def detect():
        # the scan's result is a declined plan: the flat launch that follows
        # is the one already uploaded
        plan = pdk.CascadePlan(b.indptr, b.indices, b.kv_len, b.page_size, gate_params)
        assert plan.stats()[1] != "none"

    cache = pdk.PlanCache(2)
    def lookup():
        cache.get(b.indptr, b.indices, b.kv_len, b.page_size, gate_params)

    # the arms' regions interleave (the order rotating from rep to rep), so
    # that clock and thermal drift over the run falls on every arm alike
    spec = (("flat_only", []), ("detect_then_flat", [detect]),
            ("plan_cache_then_flat", [lookup]))
    for _, pre in spec:
        for _ in range(args.warmup):
            for f in pre + parts:
                f()
    region_us = {name: [] for name, _ in spec}
    for rep in range(args.reps):
        for k in range(len(spec)):
            name, pre = spec[(rep + k) % len(spec)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                for f in pre + parts:
                    f()
            torch.cuda.synchronize()
            region_us[name].append((time.perf_counter() - t0) * 1e6 / args.steps)
    arms = {name: stats_of(v) for name, v in region_us.items()}
    t0 = time.perf_counter()
    for _ in range(50):
        detect()
    detect_us = (time.perf_counter() - t0) * 1e6 / 50
    flat = arms["flat_only"]["median"]
    return {"workload": "llama3_8b_flat_paged_decode (nothing shared)", "decline": decline,
            "params": GATE_ARM, "us_per_step": arms,
            "detect_host_us": round(detect_us, 1),
            "overhead_us": {"detect": round(arms["detect_then_flat"]["median"] - flat, 2),
                            "plan_cache": round(arms["plan_cache_then_flat"]["median"] - flat, 2)}}


def merge_arm(args, torch, pdk, m, dev):
    """merge_states on 8192 output rows, H 32, D 128, 1..16 rows per group:
    (region us per launch, device us per launch, algorithmic bytes)."""
    v = torch.from_numpy(m.v_in).to(dev)
    l = torch.from_numpy(m.lse_in).to(dev)
    ind = torch.from_numpy(m.o_indptr).to(dev)
    M = len(m.o_indptr) - 1
    vo = torch.empty((M, v.shape[1], v.shape[2]), dtype=torch.float32, device=dev)
    lo = torch.empty((M, v.shape[1]), dtype=torch.float32, device=dev)
    region_ms, (dev_us,) = time_steps(torch, [lambda: pdk.merge_states(v, l, ind, vo, lo)],
                                      args.steps, args.warmup, args.reps)
    alg = m.v_in.nbytes + m.lse_in.nbytes + m.o_indptr.nbytes + vo.numel() * 4 + lo.numel() * 4
    return region_ms, dev_us, alg, M


def merge_summary(region_ms, dev_us, alg, M, m):
    us = statistics.median(dev_us)
    achieved = alg / (us * 1e-6) / 1e9
    return {"workload": "merge_states_m8192_h32_d128", "out_rows": M,
            "in_rows": int(m.o_indptr[-1]), "heads": 32, "head_dim": 128,
            "us_per_launch": stats_of([x * 1000 for x in region_ms]),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("merge.hip"), "kernel": "merge_kernel",
                         "kernel_us": round(us, 2), "kernel_us_reps": stats_of(dev_us),
                         "bytes_per_launch": alg}}


def mla_arm(args, torch, pdk, share, dev):
    """One GPU's share of an MLA decode: 32 requests, 128 query heads, latent
    576 (values = first 512 lanes), 16384 cached fp8 tokens in 4096-token
    chunks plus 256 new bf16 tokens. A step is the whole pipeline: chunk
    partials, suffix partials and the merges of every request's partials."""
    pre, suf = share.prefix, share.suffix
    p_pool, p_csr, q = device_batch(torch, pdk, pre, dev)
    s_pool, _, _ = device_batch(torch, pdk, suf, dev)
    plan = pdk.ChunkedPlan((pre.indptr, pre.indices, pre.kv_len), pre.page_size,
                           share.chunk_tokens, pre.partition_tokens,
                           (suf.indptr, suf.indices, suf.kv_len), suf.page_size,
                           suf.partition_tokens)
    Hq, Dv = pre.num_q_heads, pre.head_dim_v
    plan.upload(Hq, Dv, dev)
    out = torch.empty((pre.batch, Hq, Dv), dtype=torch.float32, device=dev)
    lse = torch.empty((pre.batch, Hq), dtype=torch.float32, device=dev)
    region_ms, (step_us,) = time_steps(
        torch, [lambda: plan.run(p_pool, s_pool, q, pre.sm_scale, out, lse)], args.steps,
        args.warmup, args.reps)
    # the dominant kernel on its own: the same partitions of the cached range
    S = pre.partition_tokens
    pind = pdk.partition_indptr(pre.kv_len, S)
    pind_d = torch.from_numpy(pind).to(dev)
    R = int(pind[-1])
    vp = torch.empty((R, Hq, Dv), dtype=torch.float32, device=dev)
    lp = torch.empty((R, Hq), dtype=torch.float32, device=dev)
    _, (part_us,) = time_steps(
        torch, [lambda: pdk.paged_decode_partial(p_pool, p_csr, q, pre.sm_scale, S, pind_d, R, vp,
                                                 lp)], args.steps, args.warmup, args.reps)
    tok_pre = int(pre.kv_len.sum())
    tok_suf = int(suf.kv_len.sum())
    flop_tok = 2 * Hq * (pre.head_dim_k + Dv)
    flops_step = flop_tok * (tok_pre + tok_suf)
    flops_part = flop_tok * tok_pre
    kv_bytes = pre.unique_kv_bytes() + suf.unique_kv_bytes()
    ms = statistics.median(region_ms)
    pus = statistics.median(part_us)
    tflops = flops_part / (pus * 1e-6) / 1e12
    return {"workload": "mla_decode_share_b32_ctx16384_fp8", "batch": pre.batch,
            "num_q_heads": Hq, "head_dim_k": pre.head_dim_k, "head_dim_v": Dv,
            "page_size": pre.page_size, "chunk_tokens": share.chunk_tokens,
            "partition_tokens": S, "suffix_tokens": int(suf.kv_len[0]),
            "us_per_step": round(ms * 1000, 2),
            "reps": {"us_per_step": stats_of([m * 1000 for m in region_ms])},
            "step_device_us": stats_of(step_us),
            "tflops_per_step": round(flops_step / (ms * 1e-3) / 1e12, 2),
            "frac_of_mfma_peak": round(flops_step / (ms * 1e-3) / 1e12 /
                                       MFMA_BF16_PEAK_TFLOPS, 4),
            "kv_bytes": kv_bytes, "flops_per_step": flops_step,
            "hbm_frac_of_peak": round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_record("partial_latent.hip"),
                         "mfma_busy": mfma_busy_record("partial_latent.hip"),
                         "kernel": "partial_latent_fp8_kernel<576,512>",
                         "kernel_us": round(pus, 2), "kernel_us_reps": stats_of(part_us),
                         "flops_per_launch": flops_part}}


def cascade_partial_bytes(b, plan):
    """Algorithmic HBM bytes of one cascade partial launch: every K/V byte of
    both views once (the unique KV bytes), the query rows each level reads,
    both views' page tables, and the partial states written; returns
    (total, partial-state bytes)."""
    members = len(plan.field("members"))
    Hq, D = b.num_q_heads, b.head_dim_v
    q_row = Hq * b.head_dim_k * b.q.itemsize
    rows = int(plan.field("fused_merge_indptr")[-1])
    tables = sum(plan.field(f).nbytes for f in ("l0_indptr", "l0_indices", "l0_len", "l1_indptr",
                                                 "l1_indices", "l1_len", "group_indptr",
                                                 "members"))
    states = rows * Hq * (D + 1) * 4
    return b.unique_kv_bytes() + (members + b.batch) * q_row + tables + states, states


def planning_with_device_table_us(torch, pdk, b, csr, params, reps=50):
    """Host time to plan a step whose page table lives on the GPU: (a) copy
    the page ids to the host and run the host planner, (b) device detection
    (a kernel and a two-int-per-request readback, then the host rules)."""
    pdk.CascadePlan.from_device(csr, b.indptr, b.kv_len, b.page_size, params)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        ix = csr.indices.cpu().numpy()
        plan = pdk.CascadePlan(b.indptr, ix, b.kv_len, b.page_size, params)
        del plan
    host_us = (time.perf_counter() - t0) * 1e6 / reps
    t0 = time.perf_counter()
    for _ in range(reps):
        plan = pdk.CascadePlan.from_device(csr, b.indptr, b.kv_len, b.page_size, params)
        del plan
    dev_us = (time.perf_counter() - t0) * 1e6 / reps
    return {"copy_ids_then_host_plan_us": round(host_us, 1),
            "device_detection_plan_us": round(dev_us, 1)}


def run_arms(args, torch, pdk, b, pool, q, dev, arms_spec, tune_base=None, bytes_arm=None):
    """Time each (name, params) arm on batch b; params None: the autotuner's
    choice for the shape bucket, starting from tune_base (tuned outside the
    timed steps). Returns the arms and, for bytes_arm, the algorithmic bytes
    of its partial launch. An arm's headline rate is over its cold-cache
    steps (the step a model sees, with other layers' data between two steps
    of one layer); the back-to-back rate is given beside it."""
    kv = b.unique_kv_bytes()
    arms, part = {}, (None, None)
    for name, kw in arms_spec:
        tuning = None
        if kw is None:
            t0 = time.perf_counter()
            params, info = pdk.cascade_autotune(
                b.indptr, b.indices, b.kv_len, b.page_size, params_of(pdk, tune_base), pool, q,
                b.sm_scale, [256, 512, 1024, 2048], [256, 512, 1024], reps=5)
            tuning = {"l0_partition_tokens": params.l0_partition_tokens,
                      "l1_partition_tokens": params.l1_partition_tokens,
                      "tuned_cold_us": round(info["us"], 2), "measured": info["measured"],
                      "tuning_s": round(time.perf_counter() - t0, 3)}
        else:
            params = params_of(pdk, kw)
        plan, plan_us = planned(torch, pdk, b, params, dev)
        region_ms, t_part, t_merge, cold_us = run_plan_steps(args, torch, b, pool, q, plan, dev)
        stats, decline = plan.stats()
        if name == bytes_arm:
            part = cascade_partial_bytes(b, plan)
        warm = statistics.median(region_ms) * 1000
        cold = stats_of(cold_us)
        arms[name] = {"params": kw,
                      "cold_cache_us_per_step": cold,
                      "us_per_step": stats_of([m * 1000 for m in region_ms]),
                      "unique_kv_GBps": round(kv / (cold["median"] * 1e-6) / 1e9, 2),
                      "frac_of_peak": round(kv / (cold["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                            4),
                      "back_to_back_unique_kv_GBps": round(kv / (warm * 1e-6) / 1e9, 2),
                      "back_to_back_frac_of_peak": round(kv / (warm * 1e-6) / 1e9 /
                                                         HBM_PEAK_GBS, 4),
                      "partials_us": stats_of(t_part), "merge_us": stats_of(t_merge),
                      "plan_host_us": round(plan_us, 1),
                      "plan_cache_hit_us": round(plan_cache_hit_us(pdk, b, params), 1),
                      "members": stats["members"], "tuning": tuning,
                      "spans": len(plan.field("span_pages")),
                      "shared_pages": stats["shared_pages"], "decline": decline}
        del plan
    return arms, part


def cascade_arms(args, torch, pdk, b, dev):
    """Shared-prefix workload (batch 72: 4 groups x 16 members sharing 4096
    tokens, private suffixes U[64,1024], 8 non-members of 2048 tokens): flat,
    the page's single-subgroup cascade, and every qualifying group (both
    levels in one grid, as two launches, and with the partition sizes the
    autotuner picks for the shape bucket on a cold cache)."""
    pool, csr, q = device_batch(torch, pdk, b, dev)
    arms, (part_bytes, state_bytes) = run_arms(
        args, torch, pdk, b, pool, q, dev,
        CASCADE_ARMS + (("cascade_all_groups_autotuned", None),),
        tune_base=CASCADE_TUNE_BASE, bytes_arm="cascade_all_groups")
    p_all = params_of(pdk, dict(CASCADE_ARMS)["cascade_all_groups"])
    planning = {"batch72": planning_with_device_table_us(torch, pdk, b, csr, p_all)}
    # a long-context table alone: 16 groups x 16 members sharing 16384 tokens
    import workloads as W
    ip, ix, kl = W.shared_prefix_table(1009, groups=16, members=16, prefix_tokens=16384)
    big = types.SimpleNamespace(indptr=ip, indices=ix, kv_len=kl, page_size=16)
    planning["batch264_ctx17k"] = planning_with_device_table_us(
        torch, pdk, big, pdk.DeviceCSR.from_host(ip, ix, kl, dev), p_all, reps=10)
    planning["batch264_ctx17k"]["page_ids"] = int(ip[-1])
    best = arms["cascade_all_groups"]
    achieved = part_bytes / (best["partials_us"]["median"] * 1e-6) / 1e9
    cold = lambda a: arms[a]["cold_cache_us_per_step"]["median"]
    warm = lambda a: arms[a]["us_per_step"]["median"]
    return {"workload": "cascade_shared_prefix_b72", "unique_kv_bytes": b.unique_kv_bytes(),
            "quoted": "cold-cache steps (back-to-back figures beside them)",
            "device_page_table_planning": planning,
            "partial_launch_bytes": part_bytes, "partial_state_bytes": state_bytes,
            "flat_read_bytes": b.read_kv_bytes(), "arms": arms,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_cascade.hip"),
                         "kernel": "cascade_partial_kernel (level 0 + level 1 in one grid)",
                         "kernel_us": best["partials_us"]["median"],
                         "bytes_per_launch": part_bytes},
            "level0_mfma_busy": mfma_busy_record("partial_dma.hip", "cascade_level0"),
            "speedup_all_groups": round(cold("flat") / cold("cascade_all_groups"), 3),
            "speedup_single_group": round(cold("flat") / cold("cascade_single_group"), 3),
            "speedup_all_groups_back_to_back": round(warm("flat") / warm("cascade_all_groups"),
                                                     3)}


def bench_flat(args, torch, pdk, W, dev, b):
    extras = {}
    if not args.no_extras:
        m = W.merge_microbench()
        log("merge_states")
        r = merge_arm(args, torch, pdk, m, dev)
        extras["merge"] = merge_summary(*r, m)
        del m
        log("mla share")
        extras["mla_share"] = mla_arm(args, torch, pdk, W.mla_decode_share(), dev)
        log("cascade arms")
        extras["cascade_vs_flat"] = cascade_arms(args, torch, pdk, W.cascade_shared_prefix(),
                                                 dev)
        torch.cuda.empty_cache()
    pool, csr, q = device_batch(torch, pdk, b, dev)
    plan, plan_us = planned(torch, pdk, b, params_of(pdk, FLAT_ARM), dev)
    if not args.no_extras:
        # the gate runs the headline's launch on the same device tensors, so
        # the headline follows it with no upload in between
        log("no-sharing gate")
        extras["no_sharing_gate"] = gate_arm(args, torch, pdk, b, pool, q, plan, dev)
    log("flat (headline)")
    res = flat_line(args, torch, pdk, b, pool, q, plan, plan_us, dev)
    res.update(extras)
    return res


def bench_cascade(args, torch, pdk, W, dev, b):
    """The shared-prefix workload alone: value = the all-groups cascade's
    rate over unique KV bytes on cold-cache steps."""
    cv = cascade_arms(args, torch, pdk, b, dev)
    best = cv["arms"]["cascade_all_groups"]
    ms = best["cold_cache_us_per_step"]["median"] / 1000
    return {"metric": METRIC, "value": best["unique_kv_GBps"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "cascade_shared_prefix_b72", "batch": 72, "groups": 4,
                       "members_per_group": 16, "prefix_tokens": 4096,
                       "suffix_tokens": "uniform[64,1024]", "extra_requests": 8,
                       "extra_tokens": 2048, "num_q_heads": 32, "num_kv_heads": 8,
                       "head_dim": 128, "page_size": 16},
            "us_per_step": round(ms * 1000, 2), "frac_of_peak": best["frac_of_peak"],
            "roofline": cv["roofline"], "partial_state_bytes": cv["partial_state_bytes"],
            "cascade_vs_flat": cv}


def bench_nested(args, torch, pdk, W, dev, b):
    """Nested sharing (batch 72: 4 tenants x 16 requests behind one 2048-token
    system prompt, a 2048-token sub-prefix per tenant, private suffixes
    U[64,1024], 8 unshared 2048-token requests): flat, one span level, and
    the tenant spans nested below it, the last also with autotuned sizes.
    value = the nested arm's rate over unique KV bytes on cold-cache steps."""
    pool, csr, q = device_batch(torch, pdk, b, dev)
    arms, (part_bytes, state_bytes) = run_arms(
        args, torch, pdk, b, pool, q, dev, NESTED_ARMS + (("nested_spans_autotuned", None),),
        tune_base=NESTED_TUNE_BASE, bytes_arm="nested_spans")
    best = arms["nested_spans"]
    kv = b.unique_kv_bytes()
    planning = planning_with_device_table_us(torch, pdk, b, csr,
                                             params_of(pdk, dict(NESTED_ARMS)["nested_spans"]))
    achieved = part_bytes / (best["partials_us"]["median"] * 1e-6) / 1e9
    ms = best["cold_cache_us_per_step"]["median"] / 1000
    cold = lambda a: arms[a]["cold_cache_us_per_step"]["median"]
    return {"metric": METRIC, "value": best["unique_kv_GBps"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "nested_shared_prefix_b72", "batch": 72, "tenants": 4,
                       "members_per_tenant": 16, "system_tokens": 2048, "tenant_tokens": 2048,
                       "suffix_tokens": "uniform[64,1024]", "extra_requests": 8,
                       "extra_tokens": 2048, "num_q_heads": 32, "num_kv_heads": 8,
                       "head_dim": 128, "page_size": 16},
            "us_per_step": round(ms * 1000, 2), "frac_of_peak": best["frac_of_peak"],
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_cascade.hip",
                                                   "nested_shared_prefix_b72"),
                         "kernel": "cascade_partial_kernel (spans + level 1 in one grid)",
                         "kernel_us": best["partials_us"]["median"],
                         "bytes_per_launch": part_bytes},
            "partial_state_bytes": state_bytes, "unique_kv_bytes": kv,
            "flat_read_bytes": b.read_kv_bytes(), "arms": arms,
            "device_page_table_planning": planning,
            "speedup_nested_vs_flat": round(cold("flat") / cold("nested_spans"), 3),
            "speedup_nested_vs_one_level": round(cold("one_span_level") / cold("nested_spans"),
                                                 3)}


def bench_merge(args, torch, pdk, W, dev, m):
    region_ms, dev_us, alg, M = merge_arm(args, torch, pdk, m, dev)
    s = merge_summary(region_ms, dev_us, alg, M, m)
    ms = statistics.median(region_ms)
    return {"metric": "merge_states HBM GB/s", "value": round(alg / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": s["workload"], "out_rows": M, "in_rows": s["in_rows"],
                       "heads": 32, "head_dim": 128},
            "us_per_step": round(ms * 1000, 2), "reps": {"us_per_step": s["us_per_launch"]},
            "roofline": s["roofline"]}


def bench_mla(args, torch, pdk, W, dev, share):
    s = mla_arm(args, torch, pdk, share, dev)
    return {"metric": "MLA decode share: MFMA TFLOP/s (frac of bf16 peak) + µs/step",
            "value": s["tflops_per_step"], "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(s["us_per_step"] / 1000, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 (fp8 e4m3 KV dequantized to bf16)", "data": "synthetic",
            "config": {k: s[k] for k in ("workload", "batch", "num_q_heads", "head_dim_k",
                                         "head_dim_v", "page_size", "chunk_tokens",
                                         "partition_tokens", "suffix_tokens")},
            **{k: v for k, v in s.items() if k not in ("workload", "batch")}}


def bench_flat_mt(args, torch, pdk, W, dev, b, T=4):
    """The Llama-3-8B-shaped flat workload with a step of T = 4 query tokens
    per request, causal over each range (a 4-token verification step):
    partials of every (request, partition, token, head), then one merge per
    request over the (token, head) pairs."""
    pool, csr, q = device_batch(torch, pdk, b, dev)
    S = b.partition_tokens
    pind = pdk.partition_indptr(b.kv_len, S)
    pind_d = torch.from_numpy(pind).to(dev)
    R, B, Hq, Dv = int(pind[-1]), b.batch, b.num_q_heads, b.head_dim_v
    v = torch.empty((R, T, Hq, Dv), dtype=torch.float32, device=dev)
    l = torch.empty((R, T, Hq), dtype=torch.float32, device=dev)
    out = torch.empty((B, T * Hq, Dv), dtype=torch.float32, device=dev)
    lse = torch.empty((B, T * Hq), dtype=torch.float32, device=dev)
    parts = [lambda: pdk.paged_multi_token_partial(pool, csr, q, b.sm_scale, True, S, pind_d, R,
                                                   v, l),
             lambda: pdk.merge_states(v.view(R, T * Hq, Dv), l.view(R, T * Hq), pind_d, out, lse)]
    region_ms, (t_part, t_merge) = time_steps(torch, parts, args.steps, args.warmup, args.reps)
    cold = stats_of(time_cold(torch, parts, max(args.steps, 10), dev))
    kv = b.unique_kv_bytes()
    alg = (kv + b.q.nbytes + R * T * Hq * (Dv + 1) * 4 + b.indices.nbytes + b.kv_len.nbytes
           + (B + 1) * 4)
    ms = statistics.median(region_ms)
    pus = statistics.median(t_part)
    value = kv / (ms * 1e-3) / 1e9
    achieved = alg / (pus * 1e-6) / 1e9
    return {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"llama3_8b_flat_{T}_token_causal_step", "batch": B,
                       "query_tokens": T, "causal": True, "num_q_heads": Hq,
                       "num_kv_heads": b.num_kv_heads, "head_dim": Dv,
                       "page_size": b.page_size, "partition_tokens": S,
                       "context_tokens": "uniform[1024,8192]",
                       "total_tokens": int(b.kv_len.sum()), "partitions": R},
            "us_per_step": round(ms * 1000, 2),
            "reps": {"us_per_step": stats_of([m * 1000 for m in region_ms])},
            "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
            "cold_cache": {"us_per_step": cold,
                           "unique_kv_GBps": round(kv / (cold["median"] * 1e-6) / 1e9, 2)},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_dma.hip",
                                                   f"llama3_8b_flat_{T}_token_causal_step"),
                         "kernel": f"partial_dma_kernel<128,32,3 stages,4 waves> ({T * b.group} rows per "
                                   "KV head)",
                         "kernel_us": round(pus, 2), "bytes_per_launch": alg},
            "kernels_us": {"partials": stats_of(t_part), "merge": stats_of(t_merge)}}


def bench_mla_mt(args, torch, pdk, W, dev, share, T=4):
    """The MLA decode share with a T = 4 token step: every token sees the
    whole fp8 cached prefix (chunks non-causal) and the bf16 suffix
    causally. Partitions of a whole chunk (4096 tokens) and of the whole
    suffix (256)."""
    pre, suf = share.prefix, share.suffix
    p_pool, p_csr, q = device_batch(torch, pdk, pre, dev)
    s_pool, _, _ = device_batch(torch, pdk, suf, dev)
    plan = pdk.ChunkedPlan((pre.indptr, pre.indices, pre.kv_len), pre.page_size,
                           share.chunk_tokens, pre.partition_tokens,
                           (suf.indptr, suf.indices, suf.kv_len), suf.page_size,
                           suf.partition_tokens)
    Hq, Dv = pre.num_q_heads, pre.head_dim_v
    plan.upload(T * Hq, Dv, dev)
    out = torch.empty((pre.batch, T, Hq, Dv), dtype=torch.float32, device=dev)
    lse = torch.empty((pre.batch, T, Hq), dtype=torch.float32, device=dev)
    parts = [lambda: plan.run(p_pool, s_pool, q, pre.sm_scale, out, lse)]
    region_ms, (step_us,) = time_steps(torch, parts, args.steps, args.warmup, args.reps)
    S = pre.partition_tokens
    pind = pdk.partition_indptr(pre.kv_len, S)
    pind_d = torch.from_numpy(pind).to(dev)
    R = int(pind[-1])
    vp = torch.empty((R, T, Hq, Dv), dtype=torch.float32, device=dev)
    lp = torch.empty((R, T, Hq), dtype=torch.float32, device=dev)
    _, (part_us,) = time_steps(
        torch, [lambda: pdk.paged_multi_token_partial(p_pool, p_csr, q, pre.sm_scale, False, S,
                                                      pind_d, R, vp, lp)],
        args.steps, args.warmup, args.reps)
    tok_pre = int(pre.kv_len.sum())
    flop_tok = 2 * Hq * (pre.head_dim_k + Dv)
    seen_suf = sum(T * int(n) - T * (T - 1) // 2 for n in suf.kv_len)
    flops_step = flop_tok * (T * tok_pre + seen_suf)
    flops_part = flop_tok * T * tok_pre
    ms = statistics.median(region_ms)
    pus = statistics.median(part_us)
    tflops = flops_part / (pus * 1e-6) / 1e12
    return {"metric": "MLA decode share: MFMA TFLOP/s (frac of bf16 peak) + µs/step",
            "value": round(flops_step / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 (fp8 e4m3 KV dequantized to bf16)",
            "data": "synthetic",
            "config": {"workload": "mla_decode_share_b32_ctx16384_fp8_4_token_step",
                       "batch": pre.batch, "query_tokens": T, "num_q_heads": Hq,
                       "head_dim_k": pre.head_dim_k, "head_dim_v": Dv,
                       "page_size": pre.page_size, "chunk_tokens": share.chunk_tokens,
                       "partition_tokens": pre.partition_tokens,
                       "suffix_tokens": int(suf.kv_len[0]),
                       "suffix_partition_tokens": suf.partition_tokens},
            "us_per_step": round(ms * 1000, 2),
            "reps": {"us_per_step": stats_of([m * 1000 for m in region_ms])},
            "step_device_us": stats_of(step_us),
            "flops_per_step": flops_step,
            "frac_of_mfma_peak": round(flops_step / (ms * 1e-3) / 1e12 /
                                       MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_record("partial_latent.hip",
                                                   "mla_decode_share_b32_ctx16384_fp8_4_token_step"),
                         "kernel": f"partial_latent_fp8_kernel<576,512> ({T} tokens x {Hq} heads)",
                         "kernel_us": round(pus, 2), "flops_per_launch": flops_part}}


def bench_copy(args, torch, pdk, W, dev, _=None):
    """Calibration: a plain device copy of 1 GiB (torch's copy kernel), the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 30
    x = torch.empty(n // 2, dtype=torch.bfloat16, device=dev).normal_()
    y = torch.empty_like(x)
    region_ms, (dev_us,) = time_steps(torch, [lambda: y.copy_(x)], args.steps, args.warmup,
                                      args.reps)
    us = statistics.median(dev_us)
    return {"metric": "device copy GB/s (read + write)", "value": round(2 * n / (us * 1e-6) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(statistics.median(region_ms), 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "copy_1GiB", "bytes_read": n, "bytes_written": n}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a few tens of milliseconds of warmup: the GPU's clocks settle over the
    # first ~40 ms of back-to-back steps
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed regions of exactly --steps steps each")
    ap.add_argument("--workload", default="flat",
                    choices=["flat", "cascade", "merge", "mla", "copy", "flat_mt", "mla_mt",
                             "nested"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="flat workload only: skip the merge, MLA, shared-prefix and gate "
                         "sub-measurements")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported "
              "(this path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.reps < 1:
        print("--steps and --reps must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_split_kv_v2_amd as pdk
    import workloads as W
    # host inputs, generated once (seeded)
    host = {"flat": W.llama3_8b_flat, "cascade": W.cascade_shared_prefix,
            "nested": W.nested_shared_prefix, "merge": W.merge_microbench,
            "mla": W.mla_decode_share, "copy": lambda: None,
            "flat_mt": lambda: W.with_query_tokens(W.llama3_8b_flat(), 4, 1006),
            "mla_mt": lambda: W.mla_share_with_query_tokens(
                W.mla_decode_share(partition_tokens=4096, suffix_partition_tokens=256), 4,
                1007)}[args.workload]()
    cpu = None
    if not args.no_cpu_baseline and args.workload != "copy":
        # before any GPU use: the oracle's worker processes are forked
        log("cpu baseline")
        cpu = cpu_baseline_for(args.workload, host)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pdk.lib()
    res = {"flat": bench_flat, "cascade": bench_cascade, "merge": bench_merge, "mla": bench_mla,
           "copy": bench_copy, "flat_mt": bench_flat_mt, "mla_mt": bench_mla_mt,
           "nested": bench_nested}[args.workload](args, torch, pdk, W, "cuda:0", host)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
