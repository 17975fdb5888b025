"""Benchmark: paged split-KV decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload flat|cascade|merge|mla|flat_mt|mla_mt|nested|copy]

A step is one attention layer's decode for the whole batch: every partial
launch and every merge of the path. Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts; plans (page-table
bookkeeping on the host) are built and uploaded before it, as they are
reused across a model's layers. Prints one JSON line.

``value`` is the achieved rate over the batch's unique KV bytes (each
distinct page row read once) per step; ``roofline`` reports the dominant
kernel with its duration measured by HIP events on the stream it is launched
on (one event pair around back-to-back launches of that kernel);
``cpu_baseline`` times the f64 oracle on a bounded sample of the same
workload on one host thread (10-15 s, in the line's unit).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attn: KV HBM GB/s (frac of peak) + µs/step; cascade vs flat"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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

    def mean_us(self, pairs):
        return 1000.0 * sum(self.marks[a].elapsed_time(self.marks[b]) for a, b in pairs) / len(pairs)


def time_steps(torch, parts, steps, warmup):
    """Exactly `steps` steps, synchronized on both sides, each step running
    the callables in `parts` in order with nothing else enqueued between them.
    Then, for each part, its mean device time from `steps` back-to-back calls
    of that part alone (time_launches: an event between two launches would
    add microseconds to each). Returns the wall time per step of the first
    run (ms) and those device times (us)."""
    for _ in range(warmup):
        for f in parts:
            f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for f in parts:
            f()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / steps
    return wall_ms, [time_launches(torch, f, steps) for f in parts]


def time_launches(torch, f, reps):
    """Mean device time (us) of one call of f: one HIP event pair on the
    current stream around reps back-to-back calls (no event between two
    calls, since each one adds microseconds to a short launch). The span
    includes the gaps between the launches, so this is an upper bound on the
    kernel's own duration."""
    f()
    timer = Timer(torch)
    a = timer.mark()
    for _ in range(reps):
        f()
    b = timer.mark()
    torch.cuda.synchronize()
    return timer.mean_us([(a, b)]) / reps


def time_cold(torch, parts, steps, dev):
    """Mean device time (us) of one step run after a 512 MiB device read
    (a sum) that evicts the step's data from the 256 MB last-level (MALL)
    cache, as the other layers of a model would between two decode steps of
    one layer. The read is outside the timed span; HIP events bracket the
    step's launches. A read, not a write: evicting dirty lines would charge
    their write-back to the step."""
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
    return timer.mean_us(spans)


def oracle_rate(units, run, amount, unit, scale, what, min_s=10.0, budget_s=15.0):
    """The f64 oracle as it stands, timed on one host thread over a bounded
    sample of the workload: the units (in a seeded order) are run one at a
    time, in repeated passes until at least min_s seconds have run and never
    past budget_s; value = the units' summed amount per second / scale."""
    import threadpoolctl
    order = [units[i] for i in np.random.default_rng(0).permutation(len(units))]
    done, total = 0, 0.0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        while time.perf_counter() - t0 < min_s:
            for u in order:
                run(u)
                done += 1
                total += amount(u)
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(total / dt / scale, 4), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{done} {what} ({done / len(units):.2f} passes over the workload's "
                      f"{len(units)}), f64 numpy oracle on one thread, {dt:.1f} s"}


def cpu_baseline(b):
    """The oracle's flat decode, one whole request (all heads) at a time: GB
    of KV attended per second."""
    from oracle import attention as oatt
    return oracle_rate(list(range(b.batch)), lambda r: oatt.decode_attention(b, requests=[r]),
                       lambda r: int(b.kv_len[r]) * b.kv_bytes_per_token(), "GB/s", 1e9,
                       "requests (all heads)")


def baseline_for(workload, x):
    """The oracle timed on the workload the GPU line measured (x: its
    inputs), in the line's unit."""
    from oracle import attention as oatt
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
    """Host time of a plan-cache lookup that hits (the key hashed and
    compared): what every layer after the first pays for its plan."""
    cache = pdk.PlanCache(2)
    cache.get(b.indptr, b.indices, b.kv_len, b.page_size, params)
    t0 = time.perf_counter()
    for _ in range(reps):
        cache.get(b.indptr, b.indices, b.kv_len, b.page_size, params)
    return (time.perf_counter() - t0) * 1e6 / reps


def run_plan_steps(args, torch, pdk, b, pool, q, plan, dev):
    """Timed steps of a planned decode: (wall ms per step, partials us, merge
    us, cold-cache us per step)."""
    out = torch.empty((b.batch, b.num_q_heads, b.head_dim_v), dtype=torch.float32, device=dev)
    lse = torch.empty((b.batch, b.num_q_heads), dtype=torch.float32, device=dev)
    parts = [lambda: plan.run_partials(pool, q, b.sm_scale), lambda: plan.run_merge(out, lse)]
    wall_ms, (t_part, t_merge) = time_steps(torch, parts, args.steps, args.warmup)
    cold_us = time_cold(torch, parts, args.steps, dev)
    return wall_ms, t_part, t_merge, cold_us


def bench_flat(args, torch, pdk, W, dev):
    b = W.llama3_8b_flat()
    pool, csr, q = device_batch(torch, pdk, b, dev)
    S = b.partition_tokens
    plan, plan_us = planned(torch, pdk, b, pdk.CascadeParams(enabled=0, l1_partition_tokens=S), dev)
    wall_ms, t_part, t_merge, cold_us = run_plan_steps(args, torch, pdk, b, pool, q, plan, dev)
    stats, _ = plan.stats()
    R = stats["suffix_chunks"]
    Hq, Dv = b.num_q_heads, b.head_dim_v
    kv = b.unique_kv_bytes()
    # the dominant kernel (partials): every KV byte once, the queries, the
    # page table, and the partial states it writes
    alg = (kv + b.q.nbytes + R * Hq * (Dv + 1) * 4 + b.indices.nbytes + b.kv_len.nbytes
           + (b.batch + 1) * 4)
    value = kv / (wall_ms * 1e-3) / 1e9
    achieved = alg / (t_part * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_flat_paged_decode", "batch": b.batch,
                   "num_q_heads": Hq, "num_kv_heads": b.num_kv_heads, "head_dim": Dv,
                   "page_size": b.page_size, "partition_tokens": S,
                   "context_tokens": "uniform[1024,8192]", "total_tokens": int(b.kv_len.sum()),
                   "partitions": R, "kv_dtype": "bf16", "query_dtype": "bf16",
                   "parallelism": "none (1 GPU)"},
        "us_per_step": round(wall_ms * 1000, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "unique_kv_bytes": kv,
        "plan_host_us": round(plan_us, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_record("partial_valu.hip"),
                     "kernel": "partial_valu_kernel<bf16,bf16,D128,4 rows>",
                     "kernel_us": round(t_part, 2), "bytes_per_launch": alg},
        "kernels_us": {"partials": round(t_part, 2), "merge": round(t_merge, 2)},
        "cold_cache": {"us_per_step": round(cold_us, 2),
                       "unique_kv_GBps": round(kv / (cold_us * 1e-6) / 1e9, 2)},
    }
    if not args.no_cascade:
        res["cascade_vs_flat"] = bench_cascade_arms(args, torch, pdk, W, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b)
    return res


def bench_flat_mt(args, torch, pdk, W, dev, T=4):
    """The Llama-3-8B-shaped flat workload with a step of T = 4 query tokens
    per request, causal over each range (a 4-token verification step):
    partials of every (request, partition, token, head), then one merge per
    request over the (token, head) pairs."""
    b = W.with_query_tokens(W.llama3_8b_flat(), T, 1006)
    args.inputs = b
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
    wall_ms, (t_part, t_merge) = time_steps(torch, parts, args.steps, args.warmup)
    cold_us = time_cold(torch, parts, args.steps, dev)
    kv = b.unique_kv_bytes()
    alg = (kv + b.q.nbytes + R * T * Hq * (Dv + 1) * 4 + b.indices.nbytes + b.kv_len.nbytes
           + (B + 1) * 4)
    value = kv / (wall_ms * 1e-3) / 1e9
    achieved = alg / (t_part * 1e-6) / 1e9
    return {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"llama3_8b_flat_{T}_token_causal_step", "batch": B,
                       "query_tokens": T, "causal": True, "num_q_heads": Hq,
                       "num_kv_heads": b.num_kv_heads, "head_dim": Dv,
                       "page_size": b.page_size, "partition_tokens": S,
                       "context_tokens": "uniform[1024,8192]",
                       "total_tokens": int(b.kv_len.sum()), "partitions": R},
            "us_per_step": round(wall_ms * 1000, 2),
            "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
            "cold_cache": {"us_per_step": round(cold_us, 2),
                           "unique_kv_GBps": round(kv / (cold_us * 1e-6) / 1e9, 2)},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_dma.hip",
                                                   f"llama3_8b_flat_{T}_token_causal_step"),
                         "kernel": f"partial_dma_kernel<128,32,4,4> ({T * b.group} rows per "
                                   "KV head)",
                         "kernel_us": round(t_part, 2), "bytes_per_launch": alg},
            "kernels_us": {"partials": round(t_part, 2), "merge": round(t_merge, 2)}}


def bench_mla_mt(args, torch, pdk, W, dev, T=4, partition_tokens=4096,
                 suffix_partition_tokens=256):
    """The MLA decode share with a T = 4 token step: every token sees the
    whole fp8 cached prefix (chunks non-causal) and the bf16 suffix
    causally. Partitions of a whole chunk (4096 tokens) and of the whole
    suffix (256): with four 128-row tiles per partition the grid is as wide
    as the one-token step's, and the partial states to merge (1 MB per
    partition) stay few."""
    share = W.mla_share_with_query_tokens(
        W.mla_decode_share(partition_tokens=partition_tokens,
                           suffix_partition_tokens=suffix_partition_tokens), T, 1007)
    pre, suf = share.prefix, share.suffix
    args.inputs = share
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
    wall_ms, (step_us,) = time_steps(torch, parts, args.steps, args.warmup)
    cold_us = time_cold(torch, parts, args.steps, dev)
    # the dominant kernel on its own: the same partitions of the cached range,
    # every token seeing all of it
    S = pre.partition_tokens
    pind = pdk.partition_indptr(pre.kv_len, S)
    pind_d = torch.from_numpy(pind).to(dev)
    R = int(pind[-1])
    vp = torch.empty((R, T, Hq, Dv), dtype=torch.float32, device=dev)
    lp = torch.empty((R, T, Hq), dtype=torch.float32, device=dev)
    _, (part_us,) = time_steps(
        torch, [lambda: pdk.paged_multi_token_partial(p_pool, p_csr, q, pre.sm_scale, False, S,
                                                      pind_d, R, vp, lp)],
        args.steps, args.warmup)
    tok_pre, tok_suf = int(pre.kv_len.sum()), int(suf.kv_len.sum())
    flop_tok = 2 * Hq * (pre.head_dim_k + Dv)
    # causal suffix: token t of a request sees suffix_len - T + t + 1 positions
    seen_suf = sum(T * int(n) - T * (T - 1) // 2 for n in suf.kv_len)
    flops_step = flop_tok * (T * tok_pre + seen_suf)
    flops_part = flop_tok * T * tok_pre
    kv_bytes = pre.unique_kv_bytes() + suf.unique_kv_bytes()
    return {"metric": "MLA decode share: MFMA TFLOP/s (frac of bf16 peak) + µs/step",
            "value": round(flops_step / (wall_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 (fp8 e4m3 KV dequantized to bf16)",
            "data": "synthetic",
            "config": {"workload": "mla_decode_share_b32_ctx16384_fp8_4_token_step",
                       "batch": pre.batch, "query_tokens": T, "num_q_heads": Hq,
                       "head_dim_k": pre.head_dim_k, "head_dim_v": Dv,
                       "page_size": pre.page_size, "chunk_tokens": share.chunk_tokens,
                       "partition_tokens": pre.partition_tokens,
                       "suffix_tokens": int(suf.kv_len[0]),
                       "suffix_partition_tokens": suf.partition_tokens},
            "us_per_step": round(wall_ms * 1000, 2), "step_device_us": round(step_us, 2),
            "cold_cache": {"us_per_step": round(cold_us, 2)},
            "kv_bytes": kv_bytes, "flops_per_step": flops_step,
            "frac_of_mfma_peak": round(flops_step / (wall_ms * 1e-3) / 1e12 /
                                       MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "mfma", "achieved": round(flops_part / (part_us * 1e-6) / 1e12, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops_part / (part_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_record("partial_latent.hip",
                                                   "mla_decode_share_b32_ctx16384_fp8_4_token_step"),
                         "kernel": f"partial_latent_kernel<576,512,fp8> ({T} tokens x {Hq} heads)",
                         "kernel_us": round(part_us, 2), "flops_per_launch": flops_part}}


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


def traffic_record(kernel_source, workload=None):
    """HBM bytes per launch from the committed rocprofv3 counter record of
    the kernel (under its source file name, or "<source>|<workload>" for a
    second workload of one kernel), or None when the kernel's sources have
    changed since it was taken."""
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(rec_path):
        return None
    key = kernel_source if workload is None else f"{kernel_source}|{workload}"
    rec = json.load(open(rec_path)).get(key)
    sha = kernel_source_sha(kernel_source)
    if not rec or sha is None or rec.get("source_sha256") != sha:
        return None
    return int(rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_factor"] +
               rec["write_kib_per_dispatch"] * 1024 * rec["write_factor"])


def bench_merge(args, torch, pdk, W, dev):
    """merge_states on 8192 output rows, H 32, D 128, 1..16 rows per group."""
    m = W.merge_microbench()
    args.inputs = m
    v = torch.from_numpy(m.v_in).to(dev)
    l = torch.from_numpy(m.lse_in).to(dev)
    ind = torch.from_numpy(m.o_indptr).to(dev)
    M = len(m.o_indptr) - 1
    vo = torch.empty((M, v.shape[1], v.shape[2]), dtype=torch.float32, device=dev)
    lo = torch.empty((M, v.shape[1]), dtype=torch.float32, device=dev)
    wall_ms, (dev_us,) = time_steps(torch, [lambda: pdk.merge_states(v, l, ind, vo, lo)],
                                    args.steps, args.warmup)
    alg = m.v_in.nbytes + m.lse_in.nbytes + m.o_indptr.nbytes + vo.numel() * 4 + lo.numel() * 4
    value = alg / (wall_ms * 1e-3) / 1e9
    achieved = alg / (dev_us * 1e-6) / 1e9
    return {"metric": "merge_states HBM GB/s", "value": round(value, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "merge_states_m8192_h32_d128", "out_rows": M,
                       "in_rows": int(m.o_indptr[-1]), "heads": 32, "head_dim": 128},
            "us_per_step": round(wall_ms * 1000, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("merge.hip"), "kernel": "merge_kernel",
                         "kernel_us": round(dev_us, 2), "bytes_per_launch": alg}}


def bench_mla(args, torch, pdk, W, dev):
    """One GPU's share of an MLA decode: 32 requests, 128 query heads, latent
    576 (values = first 512 lanes), 16384 cached fp8 tokens in 4096-token
    chunks (1024-token partitions) plus 256 new bf16 tokens. A step is the
    whole pipeline: chunk partials, per-chunk merge, merge across chunks,
    suffix partials and merge, final merge."""
    share = W.mla_decode_share()
    args.inputs = share
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
    wall_ms, (step_us,) = time_steps(
        torch, [lambda: plan.run(p_pool, s_pool, q, pre.sm_scale, out, lse)], args.steps,
        args.warmup)
    # the dominant kernel on its own: the same partitions of the cached range
    S = pre.partition_tokens
    pind = pdk.partition_indptr(pre.kv_len, S)
    pind_d = torch.from_numpy(pind).to(dev)
    R = int(pind[-1])
    vp = torch.empty((R, Hq, Dv), dtype=torch.float32, device=dev)
    lp = torch.empty((R, Hq), dtype=torch.float32, device=dev)
    _, (part_us,) = time_steps(
        torch, [lambda: pdk.paged_decode_partial(p_pool, p_csr, q, pre.sm_scale, S, pind_d, R, vp,
                                                 lp)], args.steps, args.warmup)
    tok_pre = int(pre.kv_len.sum())
    tok_suf = int(suf.kv_len.sum())
    flop_tok = 2 * Hq * (pre.head_dim_k + Dv)
    flops_step = flop_tok * (tok_pre + tok_suf)
    flops_part = flop_tok * tok_pre
    kv_bytes = pre.unique_kv_bytes() + suf.unique_kv_bytes()
    return {"metric": "MLA decode share: MFMA TFLOP/s (frac of bf16 peak) + µs/step",
            "value": round(flops_step / (wall_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 (fp8 e4m3 KV dequantized to bf16)",
            "data": "synthetic",
            "config": {"workload": "mla_decode_share_b32_ctx16384_fp8", "batch": pre.batch,
                       "num_q_heads": Hq, "head_dim_k": pre.head_dim_k, "head_dim_v": Dv,
                       "page_size": pre.page_size, "chunk_tokens": share.chunk_tokens,
                       "partition_tokens": S, "suffix_tokens": int(suf.kv_len[0])},
            "us_per_step": round(wall_ms * 1000, 2), "step_device_us": round(step_us, 2),
            "kv_bytes": kv_bytes,
            "hbm_frac_of_peak": round(kv_bytes / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "mfma", "achieved": round(flops_part / (part_us * 1e-6) / 1e12, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops_part / (part_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_record("partial_latent.hip"),
                         "kernel": "partial_latent_kernel<576,512,fp8>",
                         "kernel_us": round(part_us, 2), "flops_per_launch": flops_part}}


def bench_cascade(args, torch, pdk, W, dev):
    """The shared-prefix workload alone: flat vs cascade arms; value = the
    all-groups cascade's rate over unique KV bytes. Dominant kernel: the
    all-groups arm's partial launch (both levels in one grid)."""
    cv = bench_cascade_arms(args, torch, pdk, W, dev)
    best = cv["arms"]["cascade_all_groups"]
    alg, part_us = cv["partial_launch_bytes"], best["partials_us"]
    achieved = alg / (part_us * 1e-6) / 1e9
    return {"metric": METRIC, "value": best["unique_kv_GBps"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(best["us_per_step"] / 1000, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "cascade_shared_prefix_b72", "batch": 72, "groups": 4,
                       "members_per_group": 16, "prefix_tokens": 4096,
                       "suffix_tokens": "uniform[64,1024]", "extra_requests": 8,
                       "extra_tokens": 2048, "num_q_heads": 32, "num_kv_heads": 8,
                       "head_dim": 128, "page_size": 16},
            "us_per_step": best["us_per_step"], "frac_of_peak": best["frac_of_peak"],
            "cold_cache": {"us_per_step": best["cold_cache_us_per_step"],
                           "unique_kv_GBps": round(cv["unique_kv_bytes"] /
                                                   (best["cold_cache_us_per_step"] * 1e-6) / 1e9, 2)},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_cascade.hip"),
                         "kernel": "cascade_partial_kernel (level 0 + level 1 in one grid)",
                         "kernel_us": part_us, "bytes_per_launch": alg},
            "partial_state_bytes": cv["partial_state_bytes"],
            "cascade_vs_flat": cv}


def bench_copy(args, torch, pdk, W, dev):
    """Calibration: a plain device copy of 1 GiB (torch's copy kernel), the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 30
    x = torch.empty(n // 2, dtype=torch.bfloat16, device=dev).normal_()
    y = torch.empty_like(x)
    wall_ms, (dev_us,) = time_steps(torch, [lambda: y.copy_(x)], args.steps, args.warmup)
    return {"metric": "device copy GB/s (read + write)", "value": round(2 * n / (dev_us * 1e-6) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "copy_1GiB", "bytes_read": n, "bytes_written": n}}


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
    of its partial launch."""
    kv = b.unique_kv_bytes()
    arms, part = {}, (None, None)
    for name, params in arms_spec:
        tuning = None
        if params is None:
            t0 = time.perf_counter()
            params, info = pdk.cascade_autotune(
                b.indptr, b.indices, b.kv_len, b.page_size, tune_base, pool, q, b.sm_scale,
                [256, 512, 1024, 2048], [256, 512, 1024], reps=5)
            tuning = {"l0_partition_tokens": params.l0_partition_tokens,
                      "l1_partition_tokens": params.l1_partition_tokens,
                      "tuned_cold_us": round(info["us"], 2), "measured": info["measured"],
                      "tuning_s": round(time.perf_counter() - t0, 3)}
        plan, plan_us = planned(torch, pdk, b, params, dev)
        wall_ms, t_part, t_merge, cold_us = run_plan_steps(args, torch, pdk, b, pool, q, plan,
                                                           dev)
        stats, decline = plan.stats()
        if name == bytes_arm:
            part = cascade_partial_bytes(b, plan)
        arms[name] = {"us_per_step": round(wall_ms * 1000, 2),
                      "partials_us": round(t_part, 2), "merge_us": round(t_merge, 2),
                      "cold_cache_us_per_step": round(cold_us, 2),
                      "unique_kv_GBps": round(kv / (wall_ms * 1e-3) / 1e9, 2),
                      "frac_of_peak": round(kv / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "plan_host_us": round(plan_us, 1),
                      "plan_cache_hit_us": round(plan_cache_hit_us(pdk, b, params), 1),
                      "members": stats["members"], "tuning": tuning,
                      "spans": len(plan.field("span_pages")),
                      "shared_pages": stats["shared_pages"], "decline": decline}
        del plan
    return arms, part


def bench_cascade_arms(args, torch, pdk, W, dev):
    """Shared-prefix workload (batch 72: 4 groups x 16 members sharing 4096
    tokens, private suffixes U[64,1024], 8 non-members of 2048 tokens): flat,
    the page's single-subgroup cascade, and every qualifying group (both
    levels in one grid, as two launches, and with the partition sizes the
    autotuner picks for the shape bucket on a cold cache)."""
    b = W.cascade_shared_prefix()
    args.inputs = b
    pool, csr, q = device_batch(torch, pdk, b, dev)
    arms, (part_bytes, state_bytes) = run_arms(args, torch, pdk, b, pool, q, dev, (
        ("flat", pdk.CascadeParams(enabled=0, l1_partition_tokens=512)),
        ("cascade_single_group", pdk.CascadeParams(enabled=1, max_groups=1,
                                                   l0_partition_tokens=512,
                                                   l1_partition_tokens=512)),
        ("cascade_all_groups", pdk.CascadeParams(enabled=1, max_groups=0,
                                                 l0_partition_tokens=1024,
                                                 l1_partition_tokens=512)),
        ("cascade_all_groups_two_launches",
         pdk.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=256,
                           l1_partition_tokens=512, fuse_levels=0)),
        ("cascade_all_groups_autotuned", None)),
        tune_base=pdk.CascadeParams(enabled=1, max_groups=0), bytes_arm="cascade_all_groups")
    p_all = pdk.CascadeParams(enabled=1, max_groups=0, l0_partition_tokens=1024,
                              l1_partition_tokens=512)
    planning = {"batch72": planning_with_device_table_us(
        torch, pdk, b, pdk.DeviceCSR.from_host(b.indptr, b.indices, b.kv_len, dev), p_all)}
    # a long-context table alone: 16 groups x 16 members sharing 16384 tokens
    ip, ix, kl = W.shared_prefix_table(1009, groups=16, members=16, prefix_tokens=16384)
    big = types.SimpleNamespace(indptr=ip, indices=ix, kv_len=kl, page_size=16)
    planning["batch264_ctx17k"] = planning_with_device_table_us(
        torch, pdk, big, pdk.DeviceCSR.from_host(ip, ix, kl, dev), p_all, reps=10)
    planning["batch264_ctx17k"]["page_ids"] = int(ip[-1])
    return {"workload": "cascade_shared_prefix_b72", "unique_kv_bytes": b.unique_kv_bytes(),
            "device_page_table_planning": planning,
            "partial_launch_bytes": part_bytes, "partial_state_bytes": state_bytes,
            "flat_read_bytes": b.read_kv_bytes(), "arms": arms,
            "speedup_all_groups": round(arms["flat"]["us_per_step"] /
                                        arms["cascade_all_groups"]["us_per_step"], 3),
            "speedup_single_group": round(arms["flat"]["us_per_step"] /
                                          arms["cascade_single_group"]["us_per_step"], 3)}


def bench_nested(args, torch, pdk, W, dev):
    """Nested sharing (batch 72: 4 tenants x 16 requests behind one 2048-token
    system prompt, a 2048-token sub-prefix per tenant, private suffixes
    U[64,1024], 8 unshared 2048-token requests): flat, one span level (the
    system prompt; each tenant's sub-prefix read by every member), and the
    tenant spans nested below it (every shared page read once), the last with
    the sizes the autotuner picks. value = the nested arm's rate over unique
    KV bytes."""
    b = W.nested_shared_prefix()
    args.inputs = b
    pool, csr, q = device_batch(torch, pdk, b, dev)
    base = pdk.CascadeParams(enabled=1, max_groups=0, max_depth=2)
    arms, (part_bytes, state_bytes) = run_arms(args, torch, pdk, b, pool, q, dev, (
        ("flat", pdk.CascadeParams(enabled=0, l1_partition_tokens=512)),
        ("one_span_level", pdk.CascadeParams(enabled=1, max_groups=0, max_depth=1,
                                             l0_partition_tokens=1024, l1_partition_tokens=512)),
        ("nested_spans", pdk.CascadeParams(enabled=1, max_groups=0, max_depth=2,
                                           l0_partition_tokens=1024, l1_partition_tokens=512)),
        ("nested_spans_autotuned", None)), tune_base=base, bytes_arm="nested_spans")
    best = arms["nested_spans"]
    kv = b.unique_kv_bytes()
    # planning from a device page table: one detection per level of spans
    planning = planning_with_device_table_us(
        torch, pdk, b, csr, pdk.CascadeParams(enabled=1, max_groups=0, max_depth=2,
                                              l0_partition_tokens=1024, l1_partition_tokens=512))
    achieved = part_bytes / (best["partials_us"] * 1e-6) / 1e9
    return {"metric": METRIC, "value": best["unique_kv_GBps"], "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(best["us_per_step"] / 1000, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "nested_shared_prefix_b72", "batch": 72, "tenants": 4,
                       "members_per_tenant": 16, "system_tokens": 2048, "tenant_tokens": 2048,
                       "suffix_tokens": "uniform[64,1024]", "extra_requests": 8,
                       "extra_tokens": 2048, "num_q_heads": 32, "num_kv_heads": 8,
                       "head_dim": 128, "page_size": 16},
            "us_per_step": best["us_per_step"], "frac_of_peak": best["frac_of_peak"],
            "cold_cache": {"us_per_step": best["cold_cache_us_per_step"],
                           "unique_kv_GBps": round(kv / (best["cold_cache_us_per_step"] * 1e-6)
                                                   / 1e9, 2)},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic_record("partial_cascade.hip",
                                                   "nested_shared_prefix_b72"),
                         "kernel": "cascade_partial_kernel (spans + level 1 in one grid)",
                         "kernel_us": best["partials_us"],
                         "bytes_per_launch": part_bytes},
            "partial_state_bytes": state_bytes, "unique_kv_bytes": kv,
            "flat_read_bytes": b.read_kv_bytes(), "arms": arms,
            "device_page_table_planning": planning,
            "speedup_nested_vs_flat": round(arms["flat"]["us_per_step"] /
                                            best["us_per_step"], 3),
            "speedup_nested_vs_one_level": round(arms["one_span_level"]["us_per_step"] /
                                                 best["us_per_step"], 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a few tens of milliseconds of warmup: the GPU's clocks settle over the
    # first ~40 ms of back-to-back steps (shorter warmups read 5-15% slower)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="flat",
                    choices=["flat", "cascade", "merge", "mla", "copy", "flat_mt", "mla_mt",
                             "nested"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cascade", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only; --gpus {args.gpus} is not supported "
              "(this path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_split_kv_v2_amd as pdk
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pdk.lib()
    res = {"flat": bench_flat, "cascade": bench_cascade, "merge": bench_merge, "mla": bench_mla,
           "copy": bench_copy, "flat_mt": bench_flat_mt, "mla_mt": bench_mla_mt,
           "nested": bench_nested}[args.workload](args, torch, pdk, W, "cuda:0")
    if not args.no_cpu_baseline and "cpu_baseline" not in res and args.workload != "copy":
        res["cpu_baseline"] = baseline_for(args.workload, args.inputs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
