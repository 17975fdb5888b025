// Query rows of a partial launch: which batch query a row reads, where its
// state goes, and which positions it sees. Included by the partial kernels.
//
// A workgroup serves the query rows of one (view request b, KV head h).
// Row r is (n, g) = (r / G, r % G), query head h*G + g, and row group n is
// (m, t) = (n / T, n % T): query token t (of the step's T >= 1 tokens) of
//   * member m of the view request in a stacked view (level 0, or a chunk of
//     a request's cached range): the query and the state rows are that
//     member's own [cascade-PR, "The decomposition, and the one part that is
//     not obvious": stacked heads kv*(M*G) + m*G + g map back to member m's
//     head kv*G + g];
//   * request b itself otherwise (m = 0).
// Queries are q [*, T, Hq, Dk], states [*, T, Hq, Dv]. With causal masking
// token t sits at position kv_len - T + t of the view request and sees
// positions up to its own, so a partition past it contributes the empty
// state [DCP-PR, section 3.2 figure: the new tokens' self-attention state is
// merged with the cached chunks' states].
#pragma once

#include <limits.h>
#include <stddef.h>

#include "internal.h"

namespace pdk {

// Query rows of view request b per KV head.
__device__ __forceinline__ int view_rows(const PartialArgs& a, bool stacked, int mbase, int b) {
  return (stacked ? a.member_indptr[b + 1] - mbase : 1) * a.q_tokens * a.G;
}

// Batch query row (index into q viewed as [*, Hq, Dk]) of row group n.
__device__ __forceinline__ int query_row(const PartialArgs& a, bool stacked, int mbase, int b,
                                         int n) {
  const int m = n / a.q_tokens, t = n - m * a.q_tokens;
  return (stacked ? a.members[mbase + m] : b) * a.q_tokens + t;
}

// Index of (row group n, query head `head`) of partition p in the state
// arrays v_out [*, Dv] / lse_out [*].
__device__ __forceinline__ size_t state_index(const PartialArgs& a, bool stacked, int mbase,
                                              int b, int p, int n, int head) {
  const int m = n / a.q_tokens, t = n - m * a.q_tokens;
  const int row = (stacked ? a.out_row_base[mbase + m] : a.out_row_base[b]) + p;
  return ((size_t)row * a.q_tokens + t) * a.Hq + head;
}

// Row tiles of one unit (view request partition x KV head) on one XCD. The
// hardware hands consecutive workgroups of a grid to the eight XCDs in turn,
// so blocks b, b + 8, b + 16, ... run on one XCD and share its L2; a unit's
// n_rt row tiles all read the unit's pages, so they are placed 8 blocks
// apart. Grids with several row tiles are padded to whole groups of 8 units
// (xcd_grid_blocks); a padding block gets unit >= the unit count and exits.
__host__ __device__ inline long long xcd_grid_blocks(long long units, int n_rt) {
  return n_rt == 1 ? units : (units + 7) / 8 * 8 * n_rt;
}

__device__ __forceinline__ void xcd_unit_tile(int block, int n_rt, int& unit, int& tile) {
  if (n_rt == 1) {
    unit = block;
    tile = 0;
    return;
  }
  const int group = block / (8 * n_rt), r = block - group * 8 * n_rt;
  unit = group * 8 + (r & 7);
  tile = r >> 3;
}

// Partition p of view request b: the request's first page-id index page0 and
// the token range [start, end) the partition covers. The request's page-id
// offsets are clamped to [0, nnz) and the range to its pages and length, so
// a malformed device page table (offsets outside the page ids, fewer pages
// than the length needs, a negative partition) gives wrong numbers or an
// empty range but never a read outside the page ids; the kernels read an id
// outside [0, num_blocks) as pool row 0, on every path.
__host__ __device__ inline void part_range(const PartialArgs& a, int b, int p, int& page0,
                                           int& start, int& end) {
  int lo = a.indptr[b], hi = a.indptr[b + 1];
  lo = lo < 0 ? 0 : (lo > a.nnz ? a.nnz : lo);
  hi = hi < lo ? lo : (hi > a.nnz ? a.nnz : hi);
  page0 = lo;
  const long long cap = INT_MAX / 2;
  long long s = p > 0 ? (long long)p * a.S : 0;
  s = s < cap ? s : cap;
  long long e = s + a.S;
  const long long n = a.kv_len[b], tokens = (long long)(hi - lo) * a.P;
  e = e < n ? e : n;
  e = e < tokens ? e : tokens;
  start = (int)s;
  end = (int)(e > s ? e : s);
}

// Exclusive end of the positions row group n sees (INT_MAX: the whole range).
__device__ __forceinline__ int visible_end(const PartialArgs& a, int b, int n) {
  if (!a.causal) return INT_MAX;
  return a.kv_len[b] - a.q_tokens + n % a.q_tokens + 1;
}

}  // namespace pdk
