"""Paged split-KV decode attention for MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI of ``libpdk.so`` (declared in
``include/pdk.h``). It only marshals arguments: every step of the decode
path (partials, merges, head stacking, fp8 dequant) runs in the library's
HIP kernels, and the planner runs in its C++ host code. PyTorch is used for
device memory and the current HIP stream. There is no CPU fallback: if the
library is missing or fails to load, every call raises.

Sources: mlxcel pull request "perf(core): compute shared prompt prefixes once
per decode batch" (cascade decode, merge_states contract) and ROCm/ATOM pull
request "[feat][DCP] Optimize MLA DCP (Enable Prefix Cache / Chunked Prefill
+ FP8 KVCache)" (chunked cached prefix, fp8 dequant).
"""
from __future__ import annotations

import collections
import dataclasses
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "PdkError", "lib", "KVPool", "DeviceCSR", "CascadeParams", "CascadePlan", "ChunkedPlan",
    "PlanCache", "StepGraph", "cascade_autotune", "cascade_tuned_params", "cascade_tuning_key",
    "cascade_tuning_clear",
    "partition_indptr", "validate_csr", "parse_switch", "cascade_enabled_from_env",
    "stacked_head_map", "paged_decode_partial", "merge_states", "decode_flat",
    "decode_flat_noalloc", "DECODE_FLAT_NOALLOC_MAX_BYTES",
    "paged_multi_token_partial", "multi_token_flat",
    "stack_heads", "unstack_heads", "fp8_dequant_bf16",
    "F32", "BF16", "FP8_E4M3", "DECLINE_NAMES",
]

F32, BF16, FP8_E4M3 = 0, 1, 2
DECLINE_NAMES = {0: "none", 1: "disabled", 2: "no_candidate", 3: "members_below_min",
                 4: "span_below_min", 5: "reaches_last_page"}
PLAN_FIELDS = {"members": 0, "group_indptr": 1, "span_pages": 2, "l0_indptr": 3,
               "l0_indices": 4, "l0_len": 5, "l1_indptr": 6, "l1_indices": 7, "l1_len": 8,
               "merge_indptr": 9, "fused_merge_indptr": 10, "group_of": 11, "member_rank": 12,
               "span_start": 13, "span_parent": 14}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpdk.so")
_lib = None


class PdkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pdk status {status}: {message}")
        self.status = status


class _Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


class _CSR(ctypes.Structure):
    _fields_ = [("indptr", ctypes.c_void_p), ("indices", ctypes.c_void_p),
                ("kv_len", ctypes.c_void_p), ("batch", ctypes.c_int32), ("nnz", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("min_shared_pages", ctypes.c_int32),
                ("min_members", ctypes.c_int32), ("max_groups", ctypes.c_int32),
                ("l0_partition_tokens", ctypes.c_int32), ("l1_partition_tokens", ctypes.c_int32),
                ("fuse_levels", ctypes.c_int32), ("max_depth", ctypes.c_int32)]


_P, _I, _F, _S, _L = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
_SIGS = {
    "pdk_partition_indptr": (_I, [_P, _I, _I, _P]),
    "pdk_validate_csr": (_I, [_P, _I, _I]),
    "pdk_parse_switch": (_I, [ctypes.c_char_p]),
    "pdk_cascade_enabled_from_env": (_I, [ctypes.c_char_p]),
    "pdk_stacked_head_map": (_I, [_I, _I, _I, _P]),
    "pdk_paged_decode_partial": (_I, [_P, _P, _P, _I, _I, _F, _I, _P, _I, _P, _P, _P]),
    "pdk_merge_states": (_I, [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P]),
    "pdk_decode_flat_workspace_bytes": (_S, [_I, _I, _I]),
    "pdk_decode_flat": (_I, [_P, _P, _P, _I, _I, _F, _I, _P, _I, _P, _P, _P, _S, _P]),
    "pdk_decode_flat_noalloc": (_I, [_P, _P, _P, _I, _I, _F, _I, _P, _I, _P, _P, _P]),
    "pdk_stack_heads": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P]),
    "pdk_unstack_heads": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "pdk_fp8_dequant_bf16": (_I, [_P, _L, _F, _P, _P]),
    "pdk_cascade_params_default": (None, [_P]),
    "pdk_cascade_plan_create": (_I, [_P, _I, _P, _P]),
    "pdk_cascade_plan_free": (None, [_P]),
    "pdk_cascade_plan_get": (_I, [_P, _I, _P, _P]),
    "pdk_cascade_plan_stats": (_I, [_P, _P, _P]),
    "pdk_cascade_workspace_bytes": (_S, [_P, _I, _I]),
    "pdk_cascade_plan_upload": (_I, [_P, _P, _S, _P]),
    "pdk_run_cascade_decode": (_I, [_P, _P, _P, _I, _I, _F, _P, _P, _P, _S, _P]),
    "pdk_run_cascade_partials": (_I, [_P, _P, _P, _I, _I, _F, _P, _S, _P]),
    "pdk_run_cascade_merge": (_I, [_P, _I, _I, _P, _P, _P, _S, _P]),
    "pdk_chunked_plan_create": (_I, [_P, _I, _I, _I, _P, _I, _I, _P]),
    "pdk_chunked_plan_free": (None, [_P]),
    "pdk_chunked_plan_counts": (_I, [_P, _P]),
    "pdk_chunked_workspace_bytes": (_S, [_P, _I, _I]),
    "pdk_chunked_plan_upload": (_I, [_P, _P, _S, _P]),
    "pdk_run_chunked_decode": (_I, [_P, _P, _P, _P, _I, _I, _F, _P, _P, _P, _P, _P, _S, _P]),
    "pdk_cascade_tuning_key": (_I, [_P, _I, _P, _P, _I, _I, _P]),
    "pdk_cascade_autotune_workspace_bytes": (_S, [_P, _I, _P, _P, _I, _P, _I, _I, _I]),
    "pdk_cascade_autotune": (_I, [_P, _I, _P, _P, _P, _I, _I, _F, _P, _I, _P, _I, _I, _P, _S,
                                  _P, _S, _P, _P, _P, _P, _P]),
    "pdk_cascade_tuned_params": (_I, [_P, _I, _P, _P, _I, _I, _P, _P]),
    "pdk_cascade_tuning_clear": (None, []),
    "pdk_cascade_device_detect_scratch_bytes": (_S, [_I]),
    "pdk_cascade_plan_create_device": (_I, [_P, _P, _P, _I, _P, _P, _S, _P, _P]),
    "pdk_cascade_plan_upload_device": (_I, [_P, _P, _P, _S, _P]),
    "pdk_plan_cache_create": (_I, [_I, _P]),
    "pdk_plan_cache_free": (None, [_P]),
    "pdk_plan_cache_get": (_I, [_P, _P, _I, _P, _P, _P, _P]),
    "pdk_plan_cache_stats": (_I, [_P, _P]),
    "pdk_paged_multi_token_partial": (_I, [_P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _P, _P,
                                           _P]),
    "pdk_multi_token_flat": (_I, [_P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _P, _P, _P, _S,
                                  _P]),
    "pdk_run_chunked_multi_token": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P, _S,
                                         _P]),
    "pdk_graph_begin": (_I, [_P]),
    "pdk_graph_end": (_I, [_P, _P]),
    "pdk_graph_launch": (_I, [_P, _P]),
    "pdk_graph_nodes": (_I, [_P, _P, _P]),
    "pdk_graph_free": (None, [_P]),
    "pdk_last_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded libpdk.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_split_kv_v2_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(status: int):
    if status != 0:
        raise PdkError(status, lib().pdk_last_error().decode())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to pdk must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


# --------------------------------------------------------------------------
# Pools and page tables
# --------------------------------------------------------------------------

@dataclass
class KVPool:
    """Device KV pool, HND [num_blocks, Hkv, P, D]; ``v is None`` for a latent
    pool whose values are the first ``head_dim_v`` lanes of each key row."""
    k: torch.Tensor
    v: Optional[torch.Tensor]
    head_dim_v: int
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def page_size(self) -> int:
        return int(self.k.shape[2])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    def struct(self) -> _Pool:
        """The C struct; the pool tensors must be contiguous HND
        [num_blocks, Hkv, P, D] (a strided view such as cache[:, 0] of a
        [N, 2, Hkv, P, D] tensor would be read with the wrong strides)."""
        k, v = self.k, self.v
        if k.dim() != 4 or not k.is_contiguous():
            raise ValueError(f"pool k must be a contiguous 4-D [num_blocks, Hkv, P, D] tensor "
                             f"(got shape {tuple(k.shape)}, contiguous={k.is_contiguous()})")
        if v is not None:
            if v.dim() != 4 or not v.is_contiguous():
                raise ValueError("pool v must be a contiguous 4-D [num_blocks, Hkv, P, Dv] "
                                 f"tensor (got shape {tuple(v.shape)})")
            if tuple(v.shape[:3]) != tuple(k.shape[:3]) or int(v.shape[3]) != int(self.head_dim_v):
                raise ValueError(f"pool v shape {tuple(v.shape)} does not match k "
                                 f"{tuple(k.shape)} and head_dim_v {self.head_dim_v}")
            if v.dtype != k.dtype:
                raise ValueError(f"pool k and v dtypes differ ({k.dtype}, {v.dtype})")
        return _Pool(self.k.data_ptr(), None if self.v is None else self.v.data_ptr(),
                     int(self.k.shape[0]), int(self.k.shape[2]), int(self.k.shape[1]),
                     int(self.k.shape[3]), int(self.head_dim_v), _dtype_code(self.k),
                     float(self.k_scale), float(self.v_scale))


@dataclass
class DeviceCSR:
    indptr: torch.Tensor
    indices: torch.Tensor
    kv_len: torch.Tensor

    @staticmethod
    def from_host(indptr, indices, kv_len, device="cuda"):
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        idx = np.asarray(indices, dtype=np.int32)
        if idx.size == 0:
            idx = np.zeros(1, np.int32)  # keep a valid device pointer
        return DeviceCSR(f(indptr), f(idx), f(kv_len))

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    def struct(self) -> _CSR:
        """The C struct; indptr [batch+1], indices [nnz] and kv_len [batch]
        must be contiguous 1-D int32 tensors (an int64 table would be read
        as twice as many int32 words)."""
        for name in ("indptr", "indices", "kv_len"):
            t = getattr(self, name)
            if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
                raise ValueError(f"page table {name} must be a contiguous 1-D int32 tensor "
                                 f"(got {t.dtype}, shape {tuple(t.shape)})")
        if int(self.indptr.numel()) != self.batch + 1:
            raise ValueError(f"indptr has {self.indptr.numel()} entries for batch {self.batch}")
        return _CSR(self.indptr.data_ptr(), self.indices.data_ptr(), self.kv_len.data_ptr(),
                    self.batch, int(self.indices.numel()))


def _host_csr(indptr, indices, kv_len):
    ip = np.ascontiguousarray(indptr, dtype=np.int32)
    ix = np.ascontiguousarray(indices, dtype=np.int32)
    kl = np.ascontiguousarray(kv_len, dtype=np.int32)
    keep = (ip, ix, kl)
    s = _CSR(ip.ctypes.data, ix.ctypes.data if ix.size else None, kl.ctypes.data,
             int(kl.size), int(ip[-1]) if ip.size else 0)
    return s, keep


# --------------------------------------------------------------------------
# Host-side integer work
# --------------------------------------------------------------------------

def partition_indptr(kv_len, partition_tokens: int) -> np.ndarray:
    kl = np.ascontiguousarray(kv_len, dtype=np.int32)
    out = np.zeros(kl.size + 1, dtype=np.int32)
    _check(lib().pdk_partition_indptr(_np_ptr(kl), int(kl.size), int(partition_tokens),
                                      _np_ptr(out)))
    return out


def validate_csr(indptr, indices, kv_len, page_size: int, num_blocks: int):
    s, keep = _host_csr(indptr, indices, kv_len)
    _check(lib().pdk_validate_csr(ctypes.byref(s), int(page_size), int(num_blocks)))


def parse_switch(value: Optional[str]) -> int:
    return int(lib().pdk_parse_switch(None if value is None else value.encode()))


def cascade_enabled_from_env(var: str) -> int:
    return int(lib().pdk_cascade_enabled_from_env(var.encode()))


def stacked_head_map(members: int, num_kv_heads: int, group: int) -> np.ndarray:
    out = np.zeros(members * num_kv_heads * group, dtype=np.int32)
    _check(lib().pdk_stacked_head_map(members, num_kv_heads, group, _np_ptr(out)))
    return out


# --------------------------------------------------------------------------
# GPU entry points
# --------------------------------------------------------------------------

def paged_decode_partial(pool: KVPool, csr: DeviceCSR, q: torch.Tensor, sm_scale: float,
                         partition_tokens: int, part_indptr: torch.Tensor, num_partitions: int,
                         v_part: Optional[torch.Tensor] = None,
                         lse_part: Optional[torch.Tensor] = None, stream=None):
    Hq = int(q.shape[1])
    if v_part is None:
        v_part = torch.empty((num_partitions, Hq, pool.head_dim_v), dtype=torch.float32,
                             device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_partitions, Hq), dtype=torch.float32, device=q.device)
    ps, cs = pool.struct(), csr.struct()
    _check(lib().pdk_paged_decode_partial(ctypes.byref(ps), ctypes.byref(cs), _ptr(q),
                                          _dtype_code(q), Hq, float(sm_scale),
                                          int(partition_tokens), _ptr(part_indptr),
                                          int(num_partitions), _ptr(v_part), _ptr(lse_part),
                                          _stream(stream)))
    return v_part, lse_part


def merge_states(v_in: torch.Tensor, lse_in: torch.Tensor, o_indptr: torch.Tensor,
                 v_out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                 stream=None, want_lse: bool = True):
    M = int(o_indptr.shape[0]) - 1
    H, D = int(v_in.shape[1]), int(v_in.shape[2])
    if v_out is None:
        v_out = torch.empty((M, H, D), dtype=torch.float32, device=v_in.device)
    if lse_out is None and want_lse:
        lse_out = torch.empty((M, H), dtype=torch.float32, device=v_in.device)
    _check(lib().pdk_merge_states(_ptr(v_in), _ptr(lse_in), int(v_in.shape[0]), _ptr(o_indptr),
                                  M, H, D, _ptr(v_out), _ptr(lse_out), _stream(stream)))
    return v_out, lse_out


def decode_flat(pool: KVPool, csr: DeviceCSR, q: torch.Tensor, sm_scale: float,
                partition_tokens: int, part_indptr: torch.Tensor, num_partitions: int,
                out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
    B, Hq = int(q.shape[0]), int(q.shape[1])
    need = int(lib().pdk_decode_flat_workspace_bytes(num_partitions, Hq, pool.head_dim_v))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, pool.head_dim_v), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ps, cs = pool.struct(), csr.struct()
    _check(lib().pdk_decode_flat(ctypes.byref(ps), ctypes.byref(cs), _ptr(q), _dtype_code(q),
                                 Hq, float(sm_scale), int(partition_tokens), _ptr(part_indptr),
                                 int(num_partitions), _ptr(out), _ptr(lse_out), _ptr(workspace),
                                 int(workspace.numel()), _stream(stream)))
    return out, lse_out


DECODE_FLAT_NOALLOC_MAX_BYTES = 32 << 20


def decode_flat_noalloc(pool: KVPool, csr: DeviceCSR, q: torch.Tensor, sm_scale: float,
                        partition_tokens: int, part_indptr: torch.Tensor, num_partitions: int,
                        out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, stream=None):
    """decode_flat with the partial states in the library's static device
    array (no workspace): out [B, Hq, Dv] and lse_out [B, Hq] are the
    caller's. Calls that overlap on one device race."""
    Hq = int(q.shape[1])
    ps, cs = pool.struct(), csr.struct()
    _check(lib().pdk_decode_flat_noalloc(ctypes.byref(ps), ctypes.byref(cs), _ptr(q),
                                         _dtype_code(q), Hq, float(sm_scale),
                                         int(partition_tokens), _ptr(part_indptr),
                                         int(num_partitions), _ptr(out), _ptr(lse_out),
                                         _stream(stream)))
    return out, lse_out


def paged_multi_token_partial(pool: KVPool, csr: DeviceCSR, q: torch.Tensor, sm_scale: float,
                              causal: bool, partition_tokens: int, part_indptr: torch.Tensor,
                              num_partitions: int, v_part: Optional[torch.Tensor] = None,
                              lse_part: Optional[torch.Tensor] = None, stream=None):
    """q [B, T, Hq, Dk] -> v_part [R, T, Hq, Dv], lse_part [R, T, Hq]."""
    T, Hq = int(q.shape[1]), int(q.shape[2])
    if v_part is None:
        v_part = torch.empty((num_partitions, T, Hq, pool.head_dim_v), dtype=torch.float32,
                             device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_partitions, T, Hq), dtype=torch.float32, device=q.device)
    ps, cs = pool.struct(), csr.struct()
    _check(lib().pdk_paged_multi_token_partial(ctypes.byref(ps), ctypes.byref(cs), _ptr(q),
                                               _dtype_code(q), Hq, T, int(bool(causal)),
                                               float(sm_scale), int(partition_tokens),
                                               _ptr(part_indptr), int(num_partitions),
                                               _ptr(v_part), _ptr(lse_part), _stream(stream)))
    return v_part, lse_part


def multi_token_flat(pool: KVPool, csr: DeviceCSR, q: torch.Tensor, sm_scale: float,
                     causal: bool, partition_tokens: int, part_indptr: torch.Tensor,
                     num_partitions: int, out: Optional[torch.Tensor] = None,
                     lse_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """q [B, T, Hq, Dk] -> out [B, T, Hq, Dv], lse_out [B, T, Hq]."""
    B, T, Hq = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    need = int(lib().pdk_decode_flat_workspace_bytes(num_partitions, T * Hq, pool.head_dim_v))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, Hq, pool.head_dim_v), dtype=torch.float32, device=q.device)
    if lse_out is None:
        lse_out = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    ps, cs = pool.struct(), csr.struct()
    _check(lib().pdk_multi_token_flat(ctypes.byref(ps), ctypes.byref(cs), _ptr(q), _dtype_code(q),
                                      Hq, T, int(bool(causal)), float(sm_scale),
                                      int(partition_tokens), _ptr(part_indptr),
                                      int(num_partitions), _ptr(out), _ptr(lse_out),
                                      _ptr(workspace), int(workspace.numel()), _stream(stream)))
    return out, lse_out


def stack_heads(q: torch.Tensor, members: torch.Tensor, num_kv_heads: int, stream=None):
    M = int(members.numel())
    Hq, D = int(q.shape[1]), int(q.shape[2])
    G = Hq // num_kv_heads
    q0 = torch.empty((M * Hq, D), dtype=q.dtype, device=q.device)
    _check(lib().pdk_stack_heads(_ptr(q), _dtype_code(q), _ptr(members), M, num_kv_heads, G, D,
                                 _ptr(q0), _stream(stream)))
    return q0


def unstack_heads(v0: torch.Tensor, lse0: Optional[torch.Tensor], members: int,
                  num_kv_heads: int, group: int, stream=None):
    D = int(v0.shape[-1])
    Hq = num_kv_heads * group
    v = torch.empty((members, Hq, D), dtype=torch.float32, device=v0.device)
    l = None if lse0 is None else torch.empty((members, Hq), dtype=torch.float32, device=v0.device)
    _check(lib().pdk_unstack_heads(_ptr(v0), _ptr(lse0), members, num_kv_heads, group, D,
                                   _ptr(v), _ptr(l), _stream(stream)))
    return v, l


def fp8_dequant_bf16(codes: torch.Tensor, scale: float, stream=None) -> torch.Tensor:
    out = torch.empty(codes.shape, dtype=torch.int16, device=codes.device)
    _check(lib().pdk_fp8_dequant_bf16(_ptr(codes), int(codes.numel()), float(scale), _ptr(out),
                                      _stream(stream)))
    return out


# --------------------------------------------------------------------------
# Cascade decode
# --------------------------------------------------------------------------

@dataclass
class CascadeParams:
    enabled: int = -1
    min_shared_pages: int = 16
    min_members: int = 2
    max_groups: int = 1
    l0_partition_tokens: int = 256
    l1_partition_tokens: int = 512
    fuse_levels: int = 1
    max_depth: int = 1

    def struct(self) -> _Params:
        return _Params(self.enabled, self.min_shared_pages, self.min_members, self.max_groups,
                       self.l0_partition_tokens, self.l1_partition_tokens, self.fuse_levels,
                       self.max_depth)


class CascadePlan:
    """A cascade plan built by the library's C++ planner from a HOST page table."""

    def __init__(self, indptr, indices, kv_len, page_size: int, params: CascadeParams):
        s, keep = _host_csr(indptr, indices, kv_len)
        p = params.struct()
        h = ctypes.c_void_p()
        _check(lib().pdk_cascade_plan_create(ctypes.byref(s), int(page_size), ctypes.byref(p),
                                             ctypes.byref(h)))
        self._h = h
        self._owner = None
        self.params = params
        self.workspace = None

    @classmethod
    def from_device(cls, csr: "DeviceCSR", indptr_host, kv_len_host, page_size: int,
                    params: CascadeParams, stream=None):
        """Plan a device page table: detection runs on the GPU, the host
        reads back two ints per request and keeps only the row offsets and
        lengths it was given; page ids are gathered on the device at upload."""
        ip = np.ascontiguousarray(indptr_host, dtype=np.int32)
        kl = np.ascontiguousarray(kv_len_host, dtype=np.int32)
        B = int(kl.size)
        need = int(lib().pdk_cascade_device_detect_scratch_bytes(B))
        scratch = torch.empty(max(need, 256), dtype=torch.uint8, device=csr.indptr.device)
        cs, p = csr.struct(), params.struct()
        h = ctypes.c_void_p()
        _check(lib().pdk_cascade_plan_create_device(ctypes.byref(cs), ip.ctypes.data,
                                                    kl.ctypes.data, int(page_size),
                                                    ctypes.byref(p), _ptr(scratch),
                                                    int(scratch.numel()), _stream(stream),
                                                    ctypes.byref(h)))
        self = cls.__new__(cls)
        self._h = h
        self._owner = None
        self.params = params
        self.workspace = None
        self._csr_dev = csr
        return self

    @classmethod
    def _borrowed(cls, handle, params, owner):
        """A plan owned by a PlanCache (not freed by this object)."""
        self = cls.__new__(cls)
        self._h = handle
        self._owner = owner
        self.params = params
        self.workspace = None
        return self

    def __del__(self):
        if getattr(self, "_h", None) and getattr(self, "_owner", None) is None and \
                _lib is not None:
            _lib.pdk_cascade_plan_free(self._h)
            self._h = None

    def field(self, name: str) -> np.ndarray:
        data = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        _check(lib().pdk_cascade_plan_get(self._h, PLAN_FIELDS[name], ctypes.byref(data),
                                          ctypes.byref(n)))
        return np.ctypeslib.as_array(data, shape=(n.value,)).copy() if n.value else \
            np.zeros(0, np.int32)

    def stats(self):
        st = (ctypes.c_int32 * 6)()
        dec = ctypes.c_int32()
        _check(lib().pdk_cascade_plan_stats(self._h, st, ctypes.byref(dec)))
        keys = ("batch", "members", "shared_pages", "shared_tokens", "prefix_chunks",
                "suffix_chunks")
        return dict(zip(keys, list(st))), DECLINE_NAMES[dec.value]

    def workspace_bytes(self, num_q_heads: int, head_dim_v: int) -> int:
        return int(lib().pdk_cascade_workspace_bytes(self._h, num_q_heads, head_dim_v))

    def upload(self, num_q_heads: int, head_dim_v: int, device="cuda", stream=None,
               workspace: Optional[torch.Tensor] = None):
        need = self.workspace_bytes(num_q_heads, head_dim_v)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        if getattr(self, "_csr_dev", None) is not None:
            cs = self._csr_dev.struct()
            _check(lib().pdk_cascade_plan_upload_device(self._h, ctypes.byref(cs),
                                                        _ptr(workspace), int(workspace.numel()),
                                                        _stream(stream)))
        else:
            _check(lib().pdk_cascade_plan_upload(self._h, _ptr(workspace),
                                                 int(workspace.numel()), _stream(stream)))
        self.workspace = workspace
        return workspace

    def run(self, pool: KVPool, q: torch.Tensor, sm_scale: float,
            out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
            stream=None):
        B, Hq = int(q.shape[0]), int(q.shape[1])
        if self.workspace is None:
            self.upload(Hq, pool.head_dim_v, q.device, stream)
        if out is None:
            out = torch.empty((B, Hq, pool.head_dim_v), dtype=torch.float32, device=q.device)
        if lse_out is None:
            lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        ps = pool.struct()
        _check(lib().pdk_run_cascade_decode(self._h, ctypes.byref(ps), _ptr(q), _dtype_code(q),
                                            Hq, float(sm_scale), _ptr(out), _ptr(lse_out),
                                            _ptr(self.workspace), int(self.workspace.numel()),
                                            _stream(stream)))
        return out, lse_out

    def run_partials(self, pool: KVPool, q: torch.Tensor, sm_scale: float, stream=None):
        """Level-0 and level-1 partial launches only (into the workspace)."""
        Hq = int(q.shape[1])
        if self.workspace is None:
            self.upload(Hq, pool.head_dim_v, q.device, stream)
        ps = pool.struct()
        _check(lib().pdk_run_cascade_partials(self._h, ctypes.byref(ps), _ptr(q), _dtype_code(q),
                                              Hq, float(sm_scale), _ptr(self.workspace),
                                              int(self.workspace.numel()), _stream(stream)))

    def run_merge(self, out: torch.Tensor, lse_out: Optional[torch.Tensor], stream=None):
        """The single merge of the workspace's partial rows into out / lse_out."""
        Hq, Dv = int(out.shape[1]), int(out.shape[2])
        _check(lib().pdk_run_cascade_merge(self._h, Hq, Dv, _ptr(out), _ptr(lse_out),
                                           _ptr(self.workspace), int(self.workspace.numel()),
                                           _stream(stream)))
        return out, lse_out


# --------------------------------------------------------------------------
# Chunked cached prefix + new suffix
# --------------------------------------------------------------------------

class _Tuning(ctypes.Structure):
    _fields_ = [("l0_partition_tokens", ctypes.c_int32), ("l1_partition_tokens", ctypes.c_int32),
                ("us", ctypes.c_float), ("measured", ctypes.c_int32)]


def _i32(values):
    a = np.ascontiguousarray(values, dtype=np.int32)
    return a, a.ctypes.data


def cascade_tuning_key(indptr, indices, kv_len, page_size: int, params: CascadeParams,
                       pool: KVPool, num_q_heads: int, q_dtype: int) -> tuple:
    s, keep = _host_csr(indptr, indices, kv_len)
    p, ps = params.struct(), pool.struct()
    key = (ctypes.c_int32 * 16)()
    _check(lib().pdk_cascade_tuning_key(ctypes.byref(s), int(page_size), ctypes.byref(p),
                                        ctypes.byref(ps), int(num_q_heads), int(q_dtype), key))
    return tuple(key)


def cascade_autotune(indptr, indices, kv_len, page_size: int, params: CascadeParams,
                     pool: KVPool, q: torch.Tensor, sm_scale: float, l0_candidates,
                     l1_candidates, reps: int = 5, flush_bytes: int = 512 << 20, stream=None):
    """Measure every (level-0, level-1) partition pair on a cold cache and
    keep the fastest for the step's shape bucket. Returns (params with the
    chosen sizes, dict with us / measured / per-candidate times)."""
    s, keep = _host_csr(indptr, indices, kv_len)
    p, ps = params.struct(), pool.struct()
    c0, p0 = _i32(l0_candidates)
    c1, p1 = _i32(l1_candidates)
    B, Hq = int(q.shape[0]), int(q.shape[1])
    Dv = pool.head_dim_v
    need = int(lib().pdk_cascade_autotune_workspace_bytes(ctypes.byref(s), int(page_size),
                                                          ctypes.byref(p), p0, len(c0), p1,
                                                          len(c1), Hq, Dv))
    if need == 0:
        raise PdkError(-1, "autotune workspace query failed (candidates or table)")
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    flush = torch.zeros(flush_bytes, dtype=torch.uint8, device=q.device) if flush_bytes else None
    out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    times = np.zeros(len(c0) * len(c1), dtype=np.float32)
    res = _Tuning()
    _check(lib().pdk_cascade_autotune(ctypes.byref(s), int(page_size), ctypes.byref(p),
                                      ctypes.byref(ps), _ptr(q), _dtype_code(q), Hq,
                                      float(sm_scale), p0, len(c0), p1, len(c1), int(reps),
                                      _ptr(flush), int(flush_bytes if flush is not None else 0),
                                      _ptr(ws), int(ws.numel()), _ptr(out), _ptr(lse),
                                      times.ctypes.data, _stream(stream), ctypes.byref(res)))
    tuned = dataclasses.replace(params, l0_partition_tokens=res.l0_partition_tokens,
                                l1_partition_tokens=res.l1_partition_tokens)
    return tuned, {"us": float(res.us), "measured": bool(res.measured),
                   "times_us": times.reshape(len(c0), len(c1))}


def cascade_tuned_params(indptr, indices, kv_len, page_size: int, params: CascadeParams,
                         pool: KVPool, num_q_heads: int, q_dtype: int):
    """(params with the bucket's tuned sizes, found)."""
    s, keep = _host_csr(indptr, indices, kv_len)
    p, ps = params.struct(), pool.struct()
    out = _Params()
    found = ctypes.c_int32()
    _check(lib().pdk_cascade_tuned_params(ctypes.byref(s), int(page_size), ctypes.byref(p),
                                          ctypes.byref(ps), int(num_q_heads), int(q_dtype),
                                          ctypes.byref(out), ctypes.byref(found)))
    tuned = dataclasses.replace(params, l0_partition_tokens=out.l0_partition_tokens,
                                l1_partition_tokens=out.l1_partition_tokens)
    return tuned, bool(found.value)


def cascade_tuning_clear():
    lib().pdk_cascade_tuning_clear()


class PlanCache:
    """Memoized cascade plans keyed by the whole page table (rows and KV
    lengths), page size and parameters; least recently used out first. The
    plan objects it returns keep their uploaded workspace across gets."""

    def __init__(self, capacity: int = 8):
        h = ctypes.c_void_p()
        _check(lib().pdk_plan_cache_create(int(capacity), ctypes.byref(h)))
        self._h = h
        self.capacity = int(capacity)
        # the C cache's entries, mirrored in the same LRU order: entry id -> plan
        self._plans = collections.OrderedDict()

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            self._plans.clear()
            _lib.pdk_plan_cache_free(self._h)
            self._h = None

    def get(self, indptr, indices, kv_len, page_size: int, params: CascadeParams):
        """(plan, hit) for this page table."""
        s, keep = _host_csr(indptr, indices, kv_len)
        p = params.struct()
        h = ctypes.c_void_p()
        eid = ctypes.c_int64()
        hit = ctypes.c_int32()
        _check(lib().pdk_plan_cache_get(self._h, ctypes.byref(s), int(page_size), ctypes.byref(p),
                                        ctypes.byref(h), ctypes.byref(eid), ctypes.byref(hit)))
        key = eid.value
        if key in self._plans:
            self._plans.move_to_end(key)
        else:
            self._plans[key] = CascadePlan._borrowed(h, params, self)
            while len(self._plans) > self.capacity:
                self._plans.popitem(last=False)
        return self._plans[key], bool(hit.value)

    def stats(self):
        st = (ctypes.c_int64 * 5)()
        _check(lib().pdk_plan_cache_stats(self._h, st))
        return dict(zip(("lookups", "hits", "builds", "evictions", "entries"), list(st)))


class ChunkedPlan:
    def __init__(self, prefix_csr, prefix_page_size: int, chunk_tokens: int,
                 prefix_partition_tokens: int, suffix_csr, suffix_page_size: int,
                 suffix_partition_tokens: int):
        s1, k1 = _host_csr(*prefix_csr)
        s2, k2 = _host_csr(*suffix_csr)
        h = ctypes.c_void_p()
        _check(lib().pdk_chunked_plan_create(ctypes.byref(s1), int(prefix_page_size),
                                             int(chunk_tokens), int(prefix_partition_tokens),
                                             ctypes.byref(s2), int(suffix_page_size),
                                             int(suffix_partition_tokens), ctypes.byref(h)))
        self._h = h
        self.workspace = None

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pdk_chunked_plan_free(self._h)
            self._h = None

    def counts(self):
        c = (ctypes.c_int32 * 4)()
        _check(lib().pdk_chunked_plan_counts(self._h, c))
        return dict(zip(("batch", "chunks", "prefix_partitions", "suffix_partitions"), list(c)))

    def upload(self, num_q_heads: int, head_dim_v: int, device="cuda", stream=None):
        need = int(lib().pdk_chunked_workspace_bytes(self._h, num_q_heads, head_dim_v))
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        _check(lib().pdk_chunked_plan_upload(self._h, _ptr(self.workspace),
                                             int(self.workspace.numel()), _stream(stream)))
        return self.workspace

    def run(self, prefix_pool: KVPool, suffix_pool: KVPool, q: torch.Tensor, sm_scale: float,
            out=None, lse_out=None, chunk_out=None, chunk_lse=None, stream=None):
        """q [B, Hq, Dk] (one token per request) or [B, T, Hq, Dk] (a step of
        T tokens: cached chunks non-causal, suffix causal)."""
        B = int(q.shape[0])
        T, Hq = (int(q.shape[1]), int(q.shape[2])) if q.dim() == 4 else (1, int(q.shape[1]))
        Dv = prefix_pool.head_dim_v
        need = int(lib().pdk_chunked_workspace_bytes(self._h, T * Hq, Dv))
        if self.workspace is None or self.workspace.numel() < need:
            self.upload(T * Hq, Dv, q.device, stream)
        lead = (B, T, Hq) if q.dim() == 4 else (B, Hq)
        if out is None:
            out = torch.empty((*lead, Dv), dtype=torch.float32, device=q.device)
        if lse_out is None:
            lse_out = torch.empty(lead, dtype=torch.float32, device=q.device)
        p1, p2 = prefix_pool.struct(), suffix_pool.struct()
        if q.dim() == 4:
            _check(lib().pdk_run_chunked_multi_token(
                self._h, ctypes.byref(p1), ctypes.byref(p2), _ptr(q), _dtype_code(q), Hq, T,
                float(sm_scale), _ptr(out), _ptr(lse_out), _ptr(chunk_out), _ptr(chunk_lse),
                _ptr(self.workspace), int(self.workspace.numel()), _stream(stream)))
        else:
            _check(lib().pdk_run_chunked_decode(self._h, ctypes.byref(p1), ctypes.byref(p2),
                                                _ptr(q), _dtype_code(q), Hq, float(sm_scale),
                                                _ptr(out), _ptr(lse_out), _ptr(chunk_out),
                                                _ptr(chunk_lse), _ptr(self.workspace),
                                                int(self.workspace.numel()), _stream(stream)))
        return out, lse_out


# --------------------------------------------------------------------------
# Step graphs
# --------------------------------------------------------------------------

class StepGraph:
    """The kernel launches that ``fn()`` makes through the library, recorded
    once by HIP stream capture (on a side stream) and replayed with one
    launch per ``replay()``. ``fn`` must only make run calls with every plan
    uploaded and every output and workspace allocated: nothing may allocate,
    copy from the host or synchronize while it records. A replay reads the
    current contents of the buffers the calls named and writes the same
    outputs; the objects those calls used (plans, pools, tensors) must stay
    alive as long as the graph."""

    def __init__(self, fn, keep=()):
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream(device=cur.device)
        side.wait_stream(cur)
        h = ctypes.c_void_p()
        with torch.cuda.stream(side):
            _check(lib().pdk_graph_begin(_stream(side)))
            try:
                fn()
            except BaseException:
                if lib().pdk_graph_end(_stream(side), ctypes.byref(h)) == 0:
                    lib().pdk_graph_free(h)
                raise
            _check(lib().pdk_graph_end(_stream(side), ctypes.byref(h)))
        cur.wait_stream(side)
        self._h = h
        self._keep = (fn, side, *keep)

    def replay(self, stream=None):
        _check(lib().pdk_graph_launch(self._h, _stream(stream)))

    def node_counts(self):
        """(kernel nodes, other nodes) recorded."""
        k, o = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pdk_graph_nodes(self._h, ctypes.byref(k), ctypes.byref(o)))
        return k.value, o.value

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pdk_graph_free(self._h)
            self._h = None
