"""Shared-prefix detection and the two-level cascade plan (integer work).

Test infrastructure only. Written from [cascade-PR] sections "Detection reads
the page table, not the refcounts", "Task items" (items 1, 2 and 4),
"Correctness coverage" and "What I left out, and where I was unsure".

Facts the page fixes:
  * Sharing is read from the page table alone: equal pool rows at equal
    positions of two requests' page lists are the same bytes.
  * Candidates are grouped by their first page; each group's span is the
    longest common page prefix of its members; a member that diverges early
    shortens the span for the whole group rather than leaving it.
  * The subgroup chosen is the one that removes the most page reads,
    span * (members - 1); one shared level only.
  * Every shared page must be full; a span that would reach a member's last
    page, a span below the page threshold and a member count below the member
    threshold all fall back to the flat launch. Defaults: 16 pages, 2 members.
  * Level 0 is a one-request view over the shared span; level 1 is the whole
    batch with the members' shared pages removed. Members merge two states
    (level 0, level 1); non-members keep their whole range at level 1 and a
    merge group of one row.
  * The launch outcome records batch, members, shared pages, shared tokens,
    prefix chunks and suffix chunks, or the reason the cascade was declined.

Readings where the page is silent (each listed in the design notes):
  R1 members are ordered by ascending batch index; member m is the m-th.
  R2 "reaches a member's last page" means span == that member's page count;
     the group is then rejected (not trimmed).
  R3 thresholds are checked per group before selection, in the order
     member count, span, last page; the first failing check names the reason.
  R4 ties in span * (members - 1) go to the group whose first member has the
     lowest batch index.
  R5 max_groups = 1 is the page's single subgroup; max_groups = 0 takes every
     qualifying group (score descending, then first index); k > 1 takes the
     best k. Selected groups are laid out at level 0 by first-member index.
  R6 prefix_chunks = sum over groups of ceil(span * P / S0);
     suffix_chunks = sum over requests of ceil(level-1 length / S1). When the
     plan declines, level 1 is the flat batch and the prefix figures are 0.
  R7 when nothing qualifies, the reason reported is that of the best-scoring
     rejected group (ties: lowest first index), or "no candidate" when no two
     requests start on the same page.
  R8 the kill switch accepts 0/false/off/no and 1/true/on/yes, compared
     without case after trimming blanks; anything else (or unset) is the
     default, which is off.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DECLINE_NONE = "none"
DECLINE_DISABLED = "disabled"
DECLINE_NO_CANDIDATE = "no_candidate"
DECLINE_MEMBERS_BELOW_MIN = "members_below_min"
DECLINE_SPAN_BELOW_MIN = "span_below_min"
DECLINE_REACHES_LAST_PAGE = "reaches_last_page"


@dataclass
class CascadeParams:
    enabled: int = -1            # -1: the shipped default (off); 0 off; 1 on
    min_shared_pages: int = 16
    min_members: int = 2
    max_groups: int = 1
    l0_partition_tokens: int = 256
    l1_partition_tokens: int = 512


@dataclass
class Group:
    members: List[int]
    span_pages: int
    score: int
    reason: str


@dataclass
class CascadePlan:
    decline: str
    batch: int
    page_size: int
    groups: List[Group] = field(default_factory=list)   # selected, level-0 order
    members: np.ndarray = None          # concatenated member batch indices
    group_indptr: np.ndarray = None     # [K+1] offsets into members
    span_pages: np.ndarray = None       # [K]
    l0_indptr: np.ndarray = None        # [K+1]
    l0_indices: np.ndarray = None
    l0_len: np.ndarray = None           # [K] tokens
    l1_indptr: np.ndarray = None        # [B+1]
    l1_indices: np.ndarray = None
    l1_len: np.ndarray = None           # [B]
    merge_indptr: np.ndarray = None     # [B+1]: 2 rows per member, 1 otherwise
    group_of: np.ndarray = None         # [B]: level-0 group of request, -1 if none
    member_rank: np.ndarray = None      # [B]: rank within its group, -1 if none
    stats: dict = field(default_factory=dict)


def enabled_from_env(value: Optional[str]) -> int:
    """Kill-switch parse [cascade-PR, "Task items", item 4]; -1 = default."""
    if value is None:
        return -1
    v = value.strip().lower()
    if v in ("0", "false", "off", "no"):
        return 0
    if v in ("1", "true", "on", "yes"):
        return 1
    return -1


def _ceil_div(a, b):
    return -(-int(a) // int(b))


def candidate_groups(indptr, indices, kv_len, page_size, params: CascadeParams):
    """Every group of >= 2 requests with the same first page, with its span,
    score and (if rejected) the reason, ordered by first member."""
    B = len(kv_len)
    by_first = {}
    for b in range(B):
        if int(indptr[b + 1]) - int(indptr[b]) >= 1 and int(kv_len[b]) >= 1:
            by_first.setdefault(int(indices[indptr[b]]), []).append(b)
    groups = []
    for first_id, mem in by_first.items():
        if len(mem) < 2:
            continue
        mem = sorted(mem)
        npages = [int(indptr[b + 1] - indptr[b]) for b in mem]
        # longest common page prefix, position by position
        lcp = 0
        while all(lcp < n for n in npages):
            pid = int(indices[indptr[mem[0]] + lcp])
            if any(int(indices[indptr[b] + lcp]) != pid for b in mem):
                break
            lcp += 1
        # keep every shared page full
        span = min([lcp] + [int(kv_len[b]) // page_size for b in mem])
        if len(mem) < params.min_members:
            reason = DECLINE_MEMBERS_BELOW_MIN
        elif span < max(1, params.min_shared_pages):
            reason = DECLINE_SPAN_BELOW_MIN
        elif any(span == n for n in npages):
            reason = DECLINE_REACHES_LAST_PAGE
        else:
            reason = DECLINE_NONE
        groups.append(Group(members=mem, span_pages=span,
                            score=span * (len(mem) - 1), reason=reason))
    groups.sort(key=lambda g: g.members[0])
    return groups


def build_cascade_plan(indptr, indices, kv_len, page_size, params: CascadeParams) -> CascadePlan:
    """Detection plus the level-0 / level-1 split of the batch page table."""
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    B = len(kv_len)
    P = int(page_size)
    S0, S1 = int(params.l0_partition_tokens), int(params.l1_partition_tokens)
    plan = CascadePlan(decline=DECLINE_NONE, batch=B, page_size=P)

    selected: List[Group] = []
    if params.enabled != 1:
        plan.decline = DECLINE_DISABLED
    else:
        cands = candidate_groups(indptr, indices, kv_len, P, params)
        ok = [g for g in cands if g.reason == DECLINE_NONE]
        if not cands:
            plan.decline = DECLINE_NO_CANDIDATE
        elif not ok:
            worst = sorted(cands, key=lambda g: (-g.score, g.members[0]))[0]
            plan.decline = worst.reason
        else:
            ranked = sorted(ok, key=lambda g: (-g.score, g.members[0]))
            take = len(ranked) if params.max_groups == 0 else params.max_groups
            selected = sorted(ranked[:take], key=lambda g: g.members[0])

    plan.groups = selected
    K = len(selected)
    group_of = np.full(B, -1, dtype=np.int64)
    member_rank = np.full(B, -1, dtype=np.int64)
    span_of = np.zeros(B, dtype=np.int64)
    members, gptr = [], [0]
    for k, g in enumerate(selected):
        for m, b in enumerate(g.members):
            group_of[b], member_rank[b], span_of[b] = k, m, g.span_pages
        members += g.members
        gptr.append(len(members))
    plan.members = np.asarray(members, dtype=np.int32)
    plan.group_indptr = np.asarray(gptr, dtype=np.int32)
    plan.span_pages = np.asarray([g.span_pages for g in selected], dtype=np.int32)
    plan.group_of = group_of.astype(np.int32)
    plan.member_rank = member_rank.astype(np.int32)

    # level 0: one request per selected group, over the span (first member's ids)
    l0_indptr, l0_idx, l0_len = [0], [], []
    for g in selected:
        b0 = g.members[0]
        l0_idx += [int(x) for x in indices[indptr[b0]:indptr[b0] + g.span_pages]]
        l0_indptr.append(len(l0_idx))
        l0_len.append(g.span_pages * P)
    plan.l0_indptr = np.asarray(l0_indptr, dtype=np.int32)
    plan.l0_indices = np.asarray(l0_idx, dtype=np.int32)
    plan.l0_len = np.asarray(l0_len, dtype=np.int32)

    # level 1: every request; members lose their first span pages
    l1_indptr, l1_idx, l1_len, merge = [0], [], [], [0]
    for b in range(B):
        s = int(span_of[b])
        l1_idx += [int(x) for x in indices[indptr[b] + s:indptr[b + 1]]]
        l1_indptr.append(len(l1_idx))
        l1_len.append(int(kv_len[b]) - s * P)
        merge.append(merge[-1] + (2 if group_of[b] >= 0 else 1))
    plan.l1_indptr = np.asarray(l1_indptr, dtype=np.int32)
    plan.l1_indices = np.asarray(l1_idx, dtype=np.int32)
    plan.l1_len = np.asarray(l1_len, dtype=np.int32)
    plan.merge_indptr = np.asarray(merge, dtype=np.int32)

    plan.stats = dict(
        batch=B,
        members=len(members),
        shared_pages=int(sum(g.span_pages for g in selected)),
        shared_tokens=int(sum(g.span_pages for g in selected)) * P,
        prefix_chunks=int(sum(_ceil_div(g.span_pages * P, S0) for g in selected)),
        suffix_chunks=int(sum(_ceil_div(n, S1) for n in l1_len)),
    )
    return plan


def stacked_head_map(num_members: int, num_kv_heads: int, group: int) -> np.ndarray:
    """KV-head-major stacking [cascade-PR, "The decomposition, and the one
    part that is not obvious"]: stacked head h0 = kv*(M*G) + m*G + g holds
    member m's query head kv*G + g. Returns, for each h0, m*Hq + (kv*G + g)."""
    M, Hkv, G = int(num_members), int(num_kv_heads), int(group)
    Hq = Hkv * G
    out = np.empty(M * Hq, dtype=np.int32)
    for kv in range(Hkv):
        for m in range(M):
            for g in range(G):
                out[kv * (M * G) + m * G + g] = m * Hq + kv * G + g
    return out


def member_major_head_map(num_members: int, num_kv_heads: int, group: int) -> np.ndarray:
    """The wrong order, h0 = m*Hq + kv*G + g (negative control only)."""
    M, Hkv, G = int(num_members), int(num_kv_heads), int(group)
    Hq = Hkv * G
    return np.arange(M * Hq, dtype=np.int32)
