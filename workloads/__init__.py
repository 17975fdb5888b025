"""Seeded synthetic inputs for paged decode attention.

This module is the only code shared by the test suite, the benchmark and the
oracle's callers. It draws random numbers and lays out page tables and paged
KV pools; it holds none of the attention, merge or planning arithmetic.
Numeric encodings (bf16, fp8 e4m3) are produced with PyTorch's own CPU dtype
conversions, so nothing here re-implements a codec that the oracle or the
kernels define.

Storage conventions (raw bytes, as a kernel sees them):
  * f32 values as ``np.float32``; bf16 as ``np.uint16`` bit patterns;
    fp8 (OCP E4M3FN) as ``np.uint8`` bit patterns.
  * KV pools are HND: ``[num_blocks, num_kv_heads, page_size, head_dim]``.
    A latent (MLA) pool has one KV head and ``v_pool is None``: V is the
    first ``head_dim_v`` lanes of each K row.
  * The page table is CSR: ``indptr[B+1]``, ``indices[nnz]`` (pool rows),
    ``kv_len[B]`` in tokens, with ``indptr[b+1]-indptr[b] == ceil(kv_len[b]/P)``.
  * Pool rows that no request references, and the slots past ``kv_len`` in a
    request's last page, hold NaN ("poison"), so a read outside the defined
    key range shows up in the output.

Seeds: the workload numbered ``i`` below draws from
``numpy.random.default_rng(1000 + i)`` (PCG64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
FP8_MAX = 448.0

DTYPES = ("f32", "bf16", "fp8_e4m3")


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """f32 -> bf16 bit patterns through torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fp8_bits(x: np.ndarray, scale: float) -> np.ndarray:
    """f32 / scale -> OCP E4M3FN bit patterns through torch's CPU conversion.

    Values are clamped to +-448 first so that no finite input maps to NaN.
    """
    y = np.clip(np.asarray(x, np.float32) / np.float32(scale), -FP8_MAX, FP8_MAX)
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


@dataclass
class PagedBatch:
    """One decode step's inputs: the queries (q [B, Hq, Dk] for one token per
    request, [B, T, Hq, Dk] for T tokens) plus a paged pool."""

    name: str
    page_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    kv_dtype: str
    q_dtype: str
    k_pool: np.ndarray
    v_pool: Optional[np.ndarray]
    indptr: np.ndarray
    indices: np.ndarray
    kv_len: np.ndarray
    q: np.ndarray
    sm_scale: float
    partition_tokens: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V that one token of one request occupies in HBM."""
        esz = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[self.kv_dtype]
        if self.v_pool is None:
            return self.num_kv_heads * self.head_dim_k * esz
        return self.num_kv_heads * (self.head_dim_k + self.head_dim_v) * esz

    def unique_kv_bytes(self) -> int:
        """Bytes of K/V in the distinct pool rows the batch references
        (whole pages as stored up to each request's last valid token)."""
        used = {}
        for b in range(self.batch):
            ids = self.indices[self.indptr[b]:self.indptr[b + 1]]
            n = int(self.kv_len[b])
            for j, pid in enumerate(ids):
                valid = min(self.page_size, n - j * self.page_size)
                used[int(pid)] = max(used.get(int(pid), 0), valid)
        return sum(used.values()) * self.kv_bytes_per_token()

    def read_kv_bytes(self) -> int:
        """Bytes a flat launch reads: every request reads its whole range."""
        return int(self.kv_len.sum()) * self.kv_bytes_per_token()


def _encode(x: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return _bf16_bits(x)
    if dtype == "fp8_e4m3":
        return _fp8_bits(x, scale)
    raise ValueError(dtype)


def _poison_value(dtype: str):
    return {"f32": np.float32(np.nan), "bf16": BF16_NAN, "fp8_e4m3": FP8_NAN}[dtype]


def _pages(n_tokens: int, page_size: int) -> int:
    return -(-int(n_tokens) // page_size)


def make_pool(rng, num_blocks, num_kv_heads, page_size, head_dim, dtype, scale=None):
    """Random N(0,1) pool in raw storage. For fp8 the per-tensor scale is
    amax/448 unless given. Returns (raw, scale)."""
    x = _normal(rng, (num_blocks, num_kv_heads, page_size, head_dim))
    if dtype == "fp8_e4m3":
        if scale is None:
            scale = float(np.abs(x).max()) / FP8_MAX
        return _encode(x, dtype, scale), float(scale)
    return _encode(x, dtype), 1.0


def poison_pool(pool: np.ndarray, dtype: str, indptr, indices, kv_len, page_size):
    """Fill with NaN every slot that no request reads: unreferenced rows, and
    the slots of a page past the most tokens any request takes from it."""
    nanv = _poison_value(dtype)
    valid = np.zeros(pool.shape[0], dtype=np.int64)
    for b in range(len(kv_len)):
        s, e = int(indptr[b]), int(indptr[b + 1])
        if e == s:
            continue
        v = np.full(e - s, page_size, dtype=np.int64)
        v[-1] = int(kv_len[b]) - (e - s - 1) * page_size
        np.maximum.at(valid, indices[s:e], v)
    for r in np.nonzero(valid < page_size)[0]:
        pool[r, :, int(valid[r]):, :] = nanv


def csr_from_page_lists(page_lists, kv_len):
    indptr = np.zeros(len(page_lists) + 1, dtype=np.int32)
    for b, pl in enumerate(page_lists):
        indptr[b + 1] = indptr[b] + len(pl)
    indices = (np.concatenate([np.asarray(p, np.int32) for p in page_lists])
               if indptr[-1] > 0 else np.zeros(0, np.int32))
    return indptr, indices.astype(np.int32), np.asarray(kv_len, dtype=np.int32)


def paged_batch_from_lists(name, rng, page_lists_logical, kv_len, *, page_size,
                           num_q_heads, num_kv_heads, head_dim_k, head_dim_v,
                           kv_dtype, q_dtype, partition_tokens, pad_blocks=4,
                           latent=False, sm_scale=None, poison=True, fp8_scale=None):
    """Build a batch from logical page ids (any hashable ints; equal ids at
    equal positions mean shared pages). Logical ids are mapped to pool rows
    through a seeded permutation so physical adjacency carries no meaning."""
    logical = sorted({int(p) for pl in page_lists_logical for p in pl})
    num_blocks = len(logical) + pad_blocks
    rows = rng.permutation(num_blocks)[: len(logical)]
    to_row = {lp: int(r) for lp, r in zip(logical, rows)}
    page_lists = [[to_row[int(p)] for p in pl] for pl in page_lists_logical]
    indptr, indices, kv_len = csr_from_page_lists(page_lists, kv_len)
    if latent:
        k_pool, ks = make_pool(rng, num_blocks, 1, page_size, head_dim_k, kv_dtype, fp8_scale)
        v_pool, vs = None, ks
    else:
        k_pool, ks = make_pool(rng, num_blocks, num_kv_heads, page_size, head_dim_k, kv_dtype, fp8_scale)
        v_pool, vs = make_pool(rng, num_blocks, num_kv_heads, page_size, head_dim_v, kv_dtype, fp8_scale)
    if poison:
        poison_pool(k_pool, kv_dtype, indptr, indices, kv_len, page_size)
        if v_pool is not None:
            poison_pool(v_pool, kv_dtype, indptr, indices, kv_len, page_size)
    B = len(kv_len)
    q = _encode(_normal(rng, (B, num_q_heads, head_dim_k)), q_dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim_k)
    return PagedBatch(name=name, page_size=page_size, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim_k=head_dim_k,
                      head_dim_v=head_dim_v, kv_dtype=kv_dtype, q_dtype=q_dtype,
                      k_pool=k_pool, v_pool=v_pool, indptr=indptr, indices=indices,
                      kv_len=kv_len, q=q, sm_scale=float(sm_scale),
                      partition_tokens=partition_tokens, k_scale=ks, v_scale=vs)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def tiny_gqa_fp32(seed: int = 1001) -> PagedBatch:
    """Tiny GQA decode, fp32: batch 4, Hq 8, Hkv 2, D 64, page 16,
    32-token partitions. Requests 0-2 share two leading pages and own 1/2/3
    private pages; request 3 owns 4 private pages. All pages are full
    (lengths 48/64/80/64). Pool: 12 used rows + 4 NaN rows, permuted."""
    rng = np.random.default_rng(seed)
    shared = [1000, 1001]
    lists = [shared + [0], shared + [10, 11], shared + [20, 21, 22], [30, 31, 32, 33]]
    kv_len = [16 * len(pl) for pl in lists]
    return paged_batch_from_lists("tiny_gqa_fp32", rng, lists, kv_len, page_size=16,
                                  num_q_heads=8, num_kv_heads=2, head_dim_k=64,
                                  head_dim_v=64, kv_dtype="f32", q_dtype="f32",
                                  partition_tokens=32, pad_blocks=4, sm_scale=1.0 / 8.0)


def llama3_8b_flat(seed: int = 1002, batch: int = 64, min_len: int = 1024,
                   max_len: int = 8192, poison: bool = True) -> PagedBatch:
    """Llama-3-8B-shaped flat decode: Hq 32, Hkv 8, D 128, bf16 KV, page 16,
    context lengths uniform in [min_len, max_len], no sharing, 512-token
    partitions."""
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(min_len, max_len + 1, size=batch)
    lists, nxt = [], 0
    for n in kv_len:
        npg = _pages(n, 16)
        lists.append(list(range(nxt, nxt + npg)))
        nxt += npg
    return paged_batch_from_lists("llama3_8b_flat", rng, lists, kv_len, page_size=16,
                                  num_q_heads=32, num_kv_heads=8, head_dim_k=128,
                                  head_dim_v=128, kv_dtype="bf16", q_dtype="bf16",
                                  partition_tokens=512, pad_blocks=16, poison=poison)


def cascade_shared_prefix(seed: int = 1003, groups: int = 4, members: int = 16,
                          prefix_tokens: int = 4096, suffix_min: int = 64,
                          suffix_max: int = 1024, extra: int = 8,
                          extra_tokens: int = 2048, poison: bool = True) -> PagedBatch:
    """Shared-prefix decode: ``groups`` groups of ``members`` requests, each
    group sharing a ``prefix_tokens`` prefix by identical page ids, private
    suffixes uniform in [suffix_min, suffix_max] tokens, plus ``extra``
    non-member requests of ``extra_tokens`` tokens. Batch slots are a seeded
    shuffle. Same heads/D/dtype/page as the flat Llama-3-8B workload."""
    rng = np.random.default_rng(seed)
    P = 16
    assert prefix_tokens % P == 0
    seqs, nxt = [], 0
    for g in range(groups):
        pref = list(range(nxt, nxt + prefix_tokens // P))
        nxt += prefix_tokens // P
        for _ in range(members):
            suf = int(rng.integers(suffix_min, suffix_max + 1))
            npg = _pages(suf, P)
            seqs.append((pref + list(range(nxt, nxt + npg)), prefix_tokens + suf, g))
            nxt += npg
    for _ in range(extra):
        npg = _pages(extra_tokens, P)
        seqs.append((list(range(nxt, nxt + npg)), extra_tokens, -1))
        nxt += npg
    order = rng.permutation(len(seqs))
    seqs = [seqs[i] for i in order]
    batch = paged_batch_from_lists("cascade_shared_prefix", rng, [s[0] for s in seqs],
                                   [s[1] for s in seqs], page_size=P, num_q_heads=32,
                                   num_kv_heads=8, head_dim_k=128, head_dim_v=128,
                                   kv_dtype="bf16", q_dtype="bf16", partition_tokens=512,
                                   pad_blocks=16, poison=poison)
    batch.meta["group_of_slot"] = [s[2] for s in seqs]
    return batch


@dataclass
class MergeInputs:
    v_in: np.ndarray      # [N, H, D] f32
    lse_in: np.ndarray    # [N, H] f32, log2 units
    o_indptr: np.ndarray  # [M+1] int32


def merge_microbench(seed: int = 1004, M: int = 8192, H: int = 32, D: int = 128,
                     max_count: int = 16) -> MergeInputs:
    """merge_states inputs: per output row a partial count uniform in
    {1..max_count}; v_in ~ N(0,1) f32; lse_in ~ U(-4, 20) f32."""
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, max_count + 1, size=M)
    o_indptr = np.zeros(M + 1, dtype=np.int32)
    o_indptr[1:] = np.cumsum(counts)
    N = int(o_indptr[-1])
    v_in = _normal(rng, (N, H, D))
    lse_in = rng.uniform(-4.0, 20.0, size=(N, H)).astype(np.float32)
    return MergeInputs(v_in=v_in, lse_in=lse_in, o_indptr=o_indptr)


@dataclass
class MlaShare:
    """One GPU's share of an MLA decode: cached fp8 latent prefix + a bf16
    new-token suffix, both paged, one latent KV head."""
    prefix: PagedBatch
    suffix: PagedBatch
    chunk_tokens: int


def mla_decode_share(seed: int = 1005, batch: int = 32, heads: int = 128,
                     context: int = 16384, suffix_tokens: int = 256,
                     chunk_tokens: int = 4096, page_size: int = 64,
                     partition_tokens: int = 2048, suffix_partition_tokens: int = 64,
                     poison: bool = True) -> MlaShare:
    """MLA-shaped share: 128 query heads, 1 latent KV head, K dim 576
    (512 latent + 64 rope), V = first 512 dims; cached prefix in an fp8
    e4m3 pool (per-tensor scale amax/448) of page 64; suffix in a bf16 pool
    of page 64; bf16 queries; scale 1/sqrt(576). Partition sizes are launch
    parameters (whole pages), not part of the data."""
    rng = np.random.default_rng(seed)
    Dk, Dv = 576, 512
    npg = _pages(context, page_size)
    lists = [list(range(b * npg, (b + 1) * npg)) for b in range(batch)]
    prefix = paged_batch_from_lists("mla_prefix_fp8", rng, lists, [context] * batch,
                                    page_size=page_size, num_q_heads=heads, num_kv_heads=1,
                                    head_dim_k=Dk, head_dim_v=Dv, kv_dtype="fp8_e4m3",
                                    q_dtype="bf16", partition_tokens=partition_tokens,
                                    pad_blocks=8, latent=True, poison=poison)
    spg = _pages(suffix_tokens, page_size)
    slists = [list(range(b * spg, (b + 1) * spg)) for b in range(batch)]
    suffix = paged_batch_from_lists("mla_suffix_bf16", rng, slists, [suffix_tokens] * batch,
                                    page_size=page_size, num_q_heads=heads, num_kv_heads=1,
                                    head_dim_k=Dk, head_dim_v=Dv, kv_dtype="bf16",
                                    q_dtype="bf16", partition_tokens=suffix_partition_tokens,
                                    pad_blocks=4, latent=True, poison=poison)
    suffix.q = prefix.q  # one query token per sequence, shared by both ranges
    return MlaShare(prefix=prefix, suffix=suffix, chunk_tokens=chunk_tokens)


def shared_prefix_table(seed: int, groups: int, members: int, prefix_tokens: int,
                        suffix_min: int = 64, suffix_max: int = 1024, extra: int = 8,
                        extra_tokens: int = 2048, page_size: int = 16):
    """The page table alone (host indptr, indices, kv_len) of a shared-prefix
    batch shaped like cascade_shared_prefix, without a KV pool: for planning
    measurements on tables too large to fill with data. Pool rows are a
    seeded permutation of the logical pages."""
    rng = np.random.default_rng(seed)
    P = page_size
    seqs, nxt = [], 0
    for g in range(groups):
        pref = list(range(nxt, nxt + prefix_tokens // P))
        nxt += len(pref)
        for _ in range(members):
            suf = int(rng.integers(suffix_min, suffix_max + 1))
            npg = _pages(suf, P)
            seqs.append((pref + list(range(nxt, nxt + npg)), prefix_tokens + suf))
            nxt += npg
    for _ in range(extra):
        npg = _pages(extra_tokens, P)
        seqs.append((list(range(nxt, nxt + npg)), extra_tokens))
        nxt += npg
    order = rng.permutation(len(seqs))
    rows = rng.permutation(nxt)
    lists = [[int(rows[p]) for p in seqs[i][0]] for i in order]
    return csr_from_page_lists(lists, [seqs[i][1] for i in order])


def nested_shared_prefix(seed: int = 1008, tenants: int = 4, members: int = 16,
                         system_tokens: int = 2048, tenant_tokens: int = 2048,
                         suffix_min: int = 64, suffix_max: int = 1024, extra: int = 8,
                         extra_tokens: int = 2048, page_size: int = 16,
                         poison: bool = True) -> PagedBatch:
    """Nested sharing: every tenant's ``members`` requests start with the
    same ``system_tokens`` pages, then the tenant's own ``tenant_tokens``
    pages, then private suffixes U[suffix_min, suffix_max]; plus ``extra``
    non-member requests of ``extra_tokens`` tokens. Batch slots are a seeded
    shuffle. Heads, head dim, dtype and page as the flat Llama-3-8B
    workload."""
    rng = np.random.default_rng(seed)
    P = page_size
    assert system_tokens % P == 0 and tenant_tokens % P == 0
    nxt = 0
    system = list(range(nxt, nxt + system_tokens // P))
    nxt += len(system)
    seqs = []
    for t in range(tenants):
        sub = list(range(nxt, nxt + tenant_tokens // P))
        nxt += len(sub)
        for _ in range(members):
            suf = int(rng.integers(suffix_min, suffix_max + 1))
            npg = _pages(suf, P)
            seqs.append((system + sub + list(range(nxt, nxt + npg)),
                         system_tokens + tenant_tokens + suf))
            nxt += npg
    for _ in range(extra):
        npg = _pages(extra_tokens, P)
        seqs.append((list(range(nxt, nxt + npg)), extra_tokens))
        nxt += npg
    order = rng.permutation(len(seqs))
    seqs = [seqs[i] for i in order]
    return paged_batch_from_lists("nested_shared_prefix", rng, [s[0] for s in seqs],
                                  [s[1] for s in seqs], page_size=P, num_q_heads=32,
                                  num_kv_heads=8, head_dim_k=128, head_dim_v=128,
                                  kv_dtype="bf16", q_dtype="bf16", partition_tokens=512,
                                  poison=poison)


# --------------------------------------------------------------------------
# Multi-token query steps
# --------------------------------------------------------------------------

def with_query_tokens(batch: PagedBatch, q_tokens: int, seed: int) -> PagedBatch:
    """The same pool and page table with ``q_tokens`` query tokens per
    request: q [B, T, Hq, Dk] drawn N(0,1) from ``seed`` and stored in the
    batch's query dtype. The range of each request is taken to end with the
    step's new tokens (how the oracle and the kernels read it)."""
    rng = np.random.default_rng(seed)
    q = _encode(_normal(rng, (batch.batch, q_tokens, batch.num_q_heads, batch.head_dim_k)),
                batch.q_dtype)
    meta = dict(batch.meta, q_tokens=q_tokens)
    return replace(batch, name=f"{batch.name}_t{q_tokens}", q=q, meta=meta)


def mla_share_with_query_tokens(share: MlaShare, q_tokens: int, seed: int) -> MlaShare:
    """An MLA share whose step carries ``q_tokens`` query tokens per request
    (shared by the cached prefix and the new-token suffix)."""
    pre = with_query_tokens(share.prefix, q_tokens, seed)
    suf = replace(share.suffix, q=pre.q, meta=dict(share.suffix.meta, q_tokens=q_tokens))
    return MlaShare(prefix=pre, suffix=suf, chunk_tokens=share.chunk_tokens)


# --------------------------------------------------------------------------
# Small randomized batches for edge cases
# --------------------------------------------------------------------------

def random_batch(seed: int, *, batch: int, page_size: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, kv_dtype: str, q_dtype: str,
                 min_len: int, max_len: int, partition_tokens: int,
                 lens=None, share: Optional[list] = None, head_dim_v: Optional[int] = None,
                 latent: bool = False, poison: bool = True) -> PagedBatch:
    """Random lengths in [min_len, max_len] (or ``lens``); optional sharing:
    ``share`` is a list of (members, n_pages) giving requests that start with
    the same ``n_pages`` page ids."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(min_len, max_len + 1, size=batch)
    lens = [int(x) for x in lens]
    lists, nxt = [], 0
    for n in lens:
        npg = _pages(n, page_size)
        lists.append(list(range(nxt, nxt + npg)))
        nxt += npg
    for members, n_pages in (share or []):
        base = list(range(nxt, nxt + n_pages))
        nxt += n_pages
        for b in members:
            k = min(n_pages, len(lists[b]))
            lists[b][:k] = base[:k]
    return paged_batch_from_lists(f"random_{seed}", rng, lists, lens, page_size=page_size,
                                  num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                                  head_dim_k=head_dim,
                                  head_dim_v=head_dim if head_dim_v is None else head_dim_v,
                                  kv_dtype=kv_dtype, q_dtype=q_dtype,
                                  partition_tokens=partition_tokens, pad_blocks=3,
                                  latent=latent, poison=poison)
