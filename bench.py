"""Benchmark: paged split-KV decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flat|cascade|merge|mla]

A step is one attention layer's decode for the whole batch: every partial
launch and every merge launch of the path. Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts. Prints one JSON
line. ``value`` is achieved GB/s over the batch's unique KV bytes (the
algorithmic bytes: each distinct page row read once); ``roofline`` reports the
dominant kernel (the partial kernel) against the 8 TB/s HBM peak with its
launch duration measured by HIP events on the launch stream; ``cpu_baseline``
times the f64 oracle on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

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


class KernelTimer:
    """HIP events around selected launches inside the timed steps."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def wrap(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return r

    def mean_us(self, name):
        ps = self.pairs.get(name, [])
        if not ps:
            return None
        return 1000.0 * sum(s.elapsed_time(e) for s, e in ps) / len(ps)

    def clear(self):
        self.pairs = {}


def timed_steps(torch, step, steps, warmup, timer):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer.clear()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def cpu_baseline_flat(b, budget_s=15.0):
    """The f64 oracle over a bounded sample of requests (whole requests, all
    heads), reported in the same unit as the GPU value."""
    import threadpoolctl
    from oracle import attention as oatt
    order = np.random.default_rng(0).permutation(b.batch)
    done, kv_bytes = [], 0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        for r in order:
            oatt.decode_attention(b, requests=[int(r)])
            done.append(int(r))
            kv_bytes += int(b.kv_len[r]) * b.kv_bytes_per_token()
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of {b.batch} requests (all heads), f64 oracle, "
                      f"1 thread, {dt:.1f} s"}


def bench_flat(args, torch, pdk, W):
    b = W.llama3_8b_flat()
    dev = "cuda:0"
    pool, csr, q = device_batch(torch, pdk, b, dev)
    S = b.partition_tokens
    pind = pdk.partition_indptr(b.kv_len, S)
    R = int(pind[-1])
    pind_d = torch.from_numpy(pind).to(dev)
    Hq, Dv = b.num_q_heads, b.head_dim_v
    v_part = torch.empty((R, Hq, Dv), dtype=torch.float32, device=dev)
    lse_part = torch.empty((R, Hq), dtype=torch.float32, device=dev)
    out = torch.empty((b.batch, Hq, Dv), dtype=torch.float32, device=dev)
    lse = torch.empty((b.batch, Hq), dtype=torch.float32, device=dev)
    timer = KernelTimer(torch)

    def step():
        timer.wrap("partial", lambda: pdk.paged_decode_partial(pool, csr, q, b.sm_scale, S, pind_d,
                                                               R, v_part, lse_part))
        timer.wrap("merge", lambda: pdk.merge_states(v_part, lse_part, pind_d, out, lse))

    ms = timed_steps(torch, step, args.steps, args.warmup, timer)
    t_part, t_merge = timer.mean_us("partial"), timer.mean_us("merge")
    kv = b.unique_kv_bytes()
    q_bytes = b.q.nbytes
    part_bytes = R * Hq * (Dv + 1) * 4
    partial_alg = kv + q_bytes + part_bytes + b.indices.nbytes + b.kv_len.nbytes
    value = kv / (ms * 1e-3) / 1e9
    achieved = partial_alg / (t_part * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_flat_decode", "batch": b.batch, "num_q_heads": Hq,
                   "num_kv_heads": b.num_kv_heads, "head_dim": Dv, "page_size": b.page_size,
                   "partition_tokens": S, "context": "uniform[1024,8192]",
                   "total_tokens": int(b.kv_len.sum()), "partitions": R,
                   "kv_dtype": "bf16", "parallelism": "none (1 GPU)"},
        "us_per_step": round(ms * 1000, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "unique_kv_bytes": kv,
        "kernels_us": {"partial": round(t_part, 2), "merge": round(t_merge, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "partial_valu_kernel (bf16, D128, 4 rows)",
                     "bytes_per_launch": partial_alg},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_flat(b)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flat", choices=["flat"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    res = {"flat": bench_flat}[args.workload](args, torch, pdk, W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
