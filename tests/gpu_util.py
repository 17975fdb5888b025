"""Helpers for the GPU parity tests: move seeded inputs to the device and
compare with the oracle under the stated tolerance metric.

Tolerance metric: pass iff max_i |gpu_i - ref_i| / max(1, |ref_i|) <= tol.
Bars: 1e-5 for f32 KV, 2e-3 for bf16 KV (f32 accumulate), 5e-3 for fp8 KV
after the identical dequant; LSE within 1e-4 log2 units (absolute);
cascade vs flat on the GPU within 1e-5.
"""
import numpy as np
import torch

import paged_split_kv_v2_amd as pdk

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8_e4m3": 5e-3}
LSE_TOL = 1e-4


def dev_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(batch, device="cuda"):
    """(pool, csr, q) device objects for a workloads.PagedBatch."""
    pool = pdk.KVPool(k=dev_tensor(batch.k_pool, device),
                      v=None if batch.v_pool is None else dev_tensor(batch.v_pool, device),
                      head_dim_v=batch.head_dim_v, k_scale=batch.k_scale, v_scale=batch.v_scale)
    csr = pdk.DeviceCSR.from_host(batch.indptr, batch.indices, batch.kv_len, device)
    q = dev_tensor(batch.q, device)
    return pool, csr, q


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    both_inf = np.isinf(ref) & (got == ref)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(got - ref))
    return float(np.max(diff / np.maximum(1.0, np.abs(np.where(both_inf, 0.0, ref)))))


def lse_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    same_inf = np.isinf(ref) & (got == ref)
    with np.errstate(invalid="ignore"):
        d = np.abs(got - ref)
    return float(np.max(np.where(same_inf, 0.0, d))) if got.size else 0.0


def assert_close(got, ref, tol, what=""):
    e = rel_err(got, ref)
    assert np.isfinite(e) and e <= tol, f"{what}: max rel err {e:.3e} > {tol:.1e}"
    return e


def assert_lse(got, ref, what=""):
    e = lse_err(got, ref)
    assert np.isfinite(e) and e <= LSE_TOL, f"{what}: LSE err {e:.3e} > {LSE_TOL:.1e}"
    return e


def flat_decode(batch, pool, csr, q, partition_tokens=None):
    S = batch.partition_tokens if partition_tokens is None else partition_tokens
    pind = pdk.partition_indptr(batch.kv_len, S)
    pind_d = torch.from_numpy(pind).to(q.device)
    out, lse = pdk.decode_flat(pool, csr, q, batch.sm_scale, S, pind_d, int(pind[-1]))
    return out, lse, pind
