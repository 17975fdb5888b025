// Paged split-KV partial attention, vector-ALU path (gfx950, wave64).
//
// Computes, for one (request, partition, KV head) per workgroup, the
// normalized partial output and the log2-unit LSE of every query row that
// reads that KV head [cascade-PR = mlxcel pull request "perf(core): compute
// shared prompt prefixes once per decode batch", section "The decomposition,
// and the one part that is not obvious": one workgroup owns all query heads
// of one KV head for one (request, page tile) and reads each K/V element
// once for all of them; section "How the #898 merge kernel is reused": the
// partial is normalized by its own denominator and its LSE is m + log2 l].
//
// Layout of the work inside a workgroup (256 threads = 4 waves):
//   * the partition's page ids are staged once in LDS, so no K/V address
//     waits on a global load inside the loop;
//   * a "row group" is one DPP row of 16 lanes; it owns one token at a time,
//     lane j holding elements [j*E, (j+1)*E) of the K and V rows (E = D/16),
//     fetched with 8- or 16-byte loads - a row group reads a contiguous K
//     row, a wave reads four adjacent tokens of a page;
//   * each step, the 16 row groups take 4 tokens each: token
//     t0 + u*16 + rowgroup, u = 0..3, i.e. 64 consecutive tokens; the K/V
//     rows of step i+1 are requested before step i is computed, so each lane
//     keeps 16 loads in flight;
//   * tokens past the end of the range are clamped to the last valid token
//     (a valid, finite row) and masked to score -inf, so the loop has no
//     per-token branches;
//   * each lane keeps the running (max, sum, accumulator) of every owned
//     query row for the tokens its row group has seen (online softmax in
//     log2 units); the K/V elements it loaded are reused from registers for
//     every owned query row;
//   * q.k partial dots are summed across the row group with DPP
//     (quad_perm, row_half_mirror, row_mirror) - no LDS traffic;
//   * at the end the 16 row-group states are merged exactly (cross-row
//     shuffles inside a wave, then LDS across the 4 waves).
// With bf16 queries and keys the dot products use v_dot2_f32_bf16 (exact
// products, f32 accumulation). Values are widened to f32 (exact) and
// accumulated with f32 FMAs.

#pragma once

#include "device.h"
#include "internal.h"
#include "rows.h"

namespace pdk {

namespace {

constexpr int kThreads = 256;
constexpr int kRowGroups = kThreads / 16;
// tokens each row group takes per step: 4, or 2 when many query rows leave
// few registers for the two K/V tiles
template <int GM, int E>
struct TokPerRowGroup { static constexpr int value = (GM * E >= 64 && GM >= 8) ? 2 : 4; };
constexpr int kMaxPartPages = 1024;                         // page ids staged in LDS
constexpr float kLazyLog2 = 8.f;  // headroom of the lazily raised softmax maximum

enum { KV_F32 = 0, KV_BF16 = 1 };

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// K/V rows are read exactly once: non-temporal (streaming) loads.
template <int NU>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[NU]) {
  if constexpr (NU % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NU / 4; ++i) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
      w[4 * i] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
    }
  } else if constexpr (NU == 2) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    w[0] = x[0]; w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < NU; ++i) w[i] = __builtin_nontemporal_load(p + i);
  }
}

// Widen E stored elements (NU words) to f32.
template <int KT, int E, int NU>
__device__ __forceinline__ void widen(const uint32_t (&w)[NU], float (&f)[E]) {
  if constexpr (KT == KV_F32) {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = bits_f32(w[e]);
  } else {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

template <int NU, int T>
struct Tile {
  uint32_t kw[T][NU];
  uint32_t vw[T][NU];
  bool valid[T];
  int tok[T];  // position of each token (read only with causal rows)
};

// Registers of a row's query: bf16 pairs for the dot2 path, else one f32
// per element.
template <int KT, int QT, int D>
struct QueryWords {
  static constexpr int value = (KT == KV_BF16 && QT == PDK_BF16) ? D / 32 : D / 16;
};

// One step of T tokens per row group for the GM owned query rows: q.k dots
// summed over the 16-lane row group (DPP, one stage at a time across all
// values), scores of invalid (or, causal, invisible) tokens masked to -inf,
// the online softmax in log2 units with a lazily raised reference maximum
// (raised only when a score exceeds it by more than kLazyLog2), and
// acc += p * v with each stored pair of V widened just before its use.
template <int KT, int QT, int D, int GM, bool CAUSAL, int NU, int T>
__device__ __forceinline__ void valu_step(const Tile<NU, T>& X,
                                          const uint32_t (&qw)[GM][QueryWords<KT, QT, D>::value],
                                          const int (&lim)[GM], float scale_log2,
                                          float (&run_m)[GM], float (&run_l)[GM],
                                          float (&acc)[GM][D / 16]) {
  constexpr int E = D / 16;
  constexpr bool kDot2 = (KT == KV_BF16 && QT == PDK_BF16);
  constexpr int QW = QueryWords<KT, QT, D>::value;
  float s[T * GM];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    float kf[E];
    if constexpr (!kDot2) widen<KT, E, NU>(X.kw[u], kf);
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      float d = 0.f;
      if constexpr (kDot2) {
#pragma unroll
        for (int i = 0; i < QW; ++i)
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[gi][i]),
                                              __builtin_bit_cast(bf16x2_t, X.kw[u][i]), d, false);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(bits_f32(qw[gi][e]), kf[e], d);
      }
      s[u * GM + gi] = d;
    }
  }
  row16_sum_n<T * GM>(s);
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int gi = 0; gi < GM; ++gi)
      s[u * GM + gi] = (X.valid[u] && (!CAUSAL || X.tok[u] < lim[gi]))
                           ? s[u * GM + gi] * scale_log2 : -INFINITY;

  // raise the reference maxima only where a score jumped past them
  float mx[GM];
  int need = 0;
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    mx[gi] = s[gi];
#pragma unroll
    for (int u = 1; u < T; ++u) mx[gi] = fmaxf(mx[gi], s[u * GM + gi]);
    need |= mx[gi] > run_m[gi] + kLazyLog2;
  }
  if (__any(need)) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      const float mn = (mx[gi] > run_m[gi] + kLazyLog2) ? mx[gi] : run_m[gi];
      const float corr = (mn == run_m[gi]) ? 1.f : fast_exp2(run_m[gi] - mn);
      run_l[gi] *= corr;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[gi][e] *= corr;
      run_m[gi] = mn;
    }
  }
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    const float mu = (run_m[gi] == -INFINITY) ? 0.f : run_m[gi];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < T; ++u) {
      s[u * GM + gi] = fast_exp2(s[u * GM + gi] - mu);
      psum += s[u * GM + gi];
    }
    run_l[gi] += psum;
  }
#pragma unroll
  for (int u = 0; u < T; ++u) {
    if constexpr (KT == KV_F32) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float v = bits_f32(X.vw[u][e]);
#pragma unroll
        for (int gi = 0; gi < GM; ++gi) acc[gi][e] = fmaf(s[u * GM + gi], v, acc[gi][e]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const float v0 = bf16_lo(X.vw[u][i]), v1 = bf16_hi(X.vw[u][i]);
#pragma unroll
        for (int gi = 0; gi < GM; ++gi) {
          acc[gi][2 * i] = fmaf(s[u * GM + gi], v0, acc[gi][2 * i]);
          acc[gi][2 * i + 1] = fmaf(s[u * GM + gi], v1, acc[gi][2 * i + 1]);
        }
      }
    }
  }
}

// Exact merge of the four row groups of a wave (lanes l, l^16, l^32, l^48):
// every lane leaves with the wave's (max, sum, accumulator) of each row.
template <int GM, int E>
__device__ __forceinline__ void valu_wave_merge(float (&run_m)[GM], float (&run_l)[GM],
                                                float (&acc)[GM][E]) {
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    float mw = fmaxf(run_m[gi], __shfl_xor(run_m[gi], 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    const float mu = (mw == -INFINITY) ? 0.f : mw;
    const float w = fast_exp2(run_m[gi] - mu);
    float l = run_l[gi] * w;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = acc[gi][e] * w;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[gi][e] = x;
    }
    run_m[gi] = mw;
    run_l[gi] = l;
  }
}

// The wave's merged states into LDS (the first row group of each wave).
template <int GM, int D>
__device__ __forceinline__ void valu_publish(float (&sm_acc)[4][GM][D], float (&sm_m)[4][GM],
                                             float (&sm_l)[4][GM], const float (&run_m)[GM],
                                             const float (&run_l)[GM],
                                             const float (&acc)[GM][D / 16]) {
  constexpr int E = D / 16;
  const int wave = threadIdx.x >> 6, j = threadIdx.x & 15;
  if ((threadIdx.x & 63) < 16) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_acc[wave][gi][j * E + e] = acc[gi][e];
      if (j == 0) {
        sm_m[wave][gi] = run_m[gi];
        sm_l[wave][gi] = run_l[gi];
      }
    }
  }
}

// Merge of the four waves' states (after a barrier) and the normalized
// partial and LSE of each of the first n_live rows: store(gi, d, value, lse)
// writes element d of row gi (lse on d == 0).
template <int GM, int D, typename Store>
__device__ __forceinline__ void valu_finish(const float (&sm_acc)[4][GM][D],
                                            const float (&sm_m)[4][GM],
                                            const float (&sm_l)[4][GM], int Dv, int n_live,
                                            Store store) {
  for (int idx = threadIdx.x; idx < GM * Dv; idx += kThreads) {
    const int gi = idx / Dv;
    const int d = idx - gi * Dv;
    if (gi >= n_live) continue;
    float M = sm_m[0][gi];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][gi]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float ww = fast_exp2(sm_m[w][gi] - Mu);
      L = fmaf(ww, sm_l[w][gi], L);
      num = fmaf(ww, sm_acc[w][gi][d], num);
    }
    store(gi, d, (L > 0.f) ? num / L : 0.f, (L > 0.f) ? M + log2f(L) : -INFINITY);
  }
}

// The LDS a workgroup of the vector body uses: the cross-wave merge of the
// row-group states and the partition's page ids. The kernel that runs the
// body owns it (a kernel running two bodies in disjoint blocks can overlay
// it on the other body's LDS).
template <int GM, int D>
struct ValuLds {
  float acc[4][GM][D];
  float m[4][GM];
  float l[4][GM];
  int pid[kMaxPartPages];
};

// The work of one workgroup of 256 threads: `block` is its index in the
// grid of its launch (the decomposition below is over that index).
template <int KT, int QT, int D, int GM, bool UNIF, bool CAUSAL>
__device__ __forceinline__ void partial_valu_body(const PartialArgs& a, const int block,
                                                  ValuLds<GM, D>& lds) {
  constexpr int E = D / 16;                          // elements per lane
  constexpr int NU = E * (KT == KV_F32 ? 4 : 2) / 4; // 32-bit words per lane per row
  constexpr bool kDot2 = (KT == KV_BF16 && QT == PDK_BF16);
  constexpr int QW = QueryWords<KT, QT, D>::value;  // per-row query registers
  constexpr int ESZ = (KT == KV_F32) ? 4 : 2;
  constexpr int T = TokPerRowGroup<GM, E>::value;
  constexpr int kStep = 16 * T;  // tokens per step of the workgroup

  float (&sm_acc)[4][GM][D] = lds.acc;
  float (&sm_m)[4][GM] = lds.m;
  float (&sm_l)[4][GM] = lds.l;
  int (&sm_pid)[kMaxPartPages] = lds.pid;

  const int n_tiles = (a.max_rows + GM - 1) / GM;
  int unit, tile;
  xcd_unit_tile(block, n_tiles, unit, tile);
  if (unit >= a.num_parts * a.Hkv) return;  // grid padding (uniform)
  const int h = unit % a.Hkv;
  const int r = unit / a.Hkv;

  const int tid = threadIdx.x;
  int b = 0, p;
  if (a.work != nullptr) {
    // planned launch: item r of the (longest-first) work list
    const int2 it = a.work[r];
    b = it.x;
    p = it.y;
  } else {
    // request of partition row r: the largest b with part_indptr[b] <= r,
    // i.e. the number of b in [1, batch) with part_indptr[b] <= r (monotone);
    // each wave counts 64 candidates per load with a ballot
    for (int base = 1; base < a.batch; base += 64) {
      const int i = base + (tid & 63);
      const bool le = (i < a.batch) && (a.part_indptr[i] <= r);
      b += __popcll(__ballot(le));
    }
    p = r - a.part_indptr[b];
  }

  const bool stacked = a.member_indptr != nullptr;
  const int mbase = stacked ? a.member_indptr[b] : 0;
  const int nrows = view_rows(a, stacked, mbase, b);
  const int row0 = tile * GM;
  if (row0 >= nrows) return;  // uniform over the workgroup

  int page0, start, end;
  part_range(a, b, p, page0, start, end);
  // causal rows: positions past the last owned row's end are never read
  int lim[GM];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) lim[gi] = INT_MAX;
  if constexpr (CAUSAL) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) lim[gi] = visible_end(a, b, (row0 + gi) / a.G);
    end = min(end, visible_end(a, b, (min(row0 + GM, nrows) - 1) / a.G));
  }
  const int shift = a.p_shift;  // page size is a power of two on this path

  const int rg = tid >> 4;
  const int j = tid & 15;

  // stage the partition's page ids (an id outside the pool reads row 0, as
  // on every path; see part_range)
  const int pg_first = start >> shift;
  if (end > start) {
    const int n_pg = ((end - 1) >> shift) - pg_first + 1;
    for (int i = tid; i < n_pg; i += kThreads) {
      const int pid = a.indices[page0 + pg_first + i];
      sm_pid[i] = ((unsigned)pid < (unsigned)a.num_blocks) ? pid : 0;
    }
  }

  // queries of the owned rows (zero for rows past nrows)
  uint32_t qw[GM][QW];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    const int row = row0 + gi;
#pragma unroll
    for (int i = 0; i < QW; ++i) qw[gi][i] = 0;
    if (row < nrows) {
      const int m = row / a.G, g = row % a.G;
      const int qb = query_row(a, stacked, mbase, b, m);
      const size_t qoff = ((size_t)qb * a.Hq + h * a.G + g) * a.Dk + j * E;
      if constexpr (QT == PDK_F32) {
        const float* qp = reinterpret_cast<const float*>(a.q) + qoff;
#pragma unroll
        for (int e = 0; e < E; ++e) qw[gi][e] = f32_bits(qp[e]);
      } else {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qoff;
        if constexpr (kDot2) {
#pragma unroll
          for (int i = 0; i < QW; ++i)
            qw[gi][i] = (uint32_t)qp[2 * i] | ((uint32_t)qp[2 * i + 1] << 16);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) qw[gi][e] = (uint32_t)qp[e] << 16;
        }
      }
    }
  }

  // running state; run_m is a reference maximum that is only raised when a
  // score exceeds it by more than kLazyLog2, so weights stay <= 2^kLazyLog2
  float run_m[GM], run_l[GM], acc[GM][E];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    run_m[gi] = -INFINITY;
    run_l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[gi][e] = 0.f;
  }

  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride * ESZ;
  const bool latent = a.v == nullptr;
  const char* vbase = latent ? kbase
                             : reinterpret_cast<const char*>(a.v) + (size_t)h * a.v_hstride * ESZ;
  const long long kb_stride = a.k_bstride * ESZ;
  const long long vb_stride = (latent ? a.k_bstride : a.v_bstride) * ESZ;
  const uint32_t krow = a.Dk * ESZ, vrow = (latent ? a.Dk : a.Dv) * ESZ;
  const uint32_t lane_off = j * NU * 4;
  const int pmask = a.P - 1;
  __syncthreads();  // page ids visible

  auto load_step = [&](int t0, Tile<NU, T>& X) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const int t = t0 + u * 16 + rg;
      const int tc = min(t, end - 1);
      int pid = sm_pid[(tc >> shift) - pg_first];
      // with pages of >= 16 tokens, the 4 tokens a wave takes for one u lie
      // in one page: its row base is wave-uniform (scalar address)
      if constexpr (UNIF) pid = __builtin_amdgcn_readfirstlane(pid);
      X.valid[u] = t < end;
      X.tok[u] = t;
      const uint32_t slot = (uint32_t)(tc & pmask);
      const char* kp = kbase + pid * kb_stride;
      const char* vp = vbase + pid * vb_stride;
      load_words<NU>(reinterpret_cast<const uint32_t*>(kp + (slot * krow + lane_off)), X.kw[u]);
      load_words<NU>(reinterpret_cast<const uint32_t*>(vp + (slot * vrow + lane_off)), X.vw[u]);
    }
  };

  auto compute_step = [&](const Tile<NU, T>& X) {
    valu_step<KT, QT, D, GM, CAUSAL>(X, qw, lim, a.scale_log2, run_m, run_l, acc);
  };

  // Two register tiles: the next step's rows are requested before the
  // current step is computed. The loop runs whole pairs of steps and the
  // last one or two steps follow it, so that every path into a step's
  // computation carries exactly the next step's loads in flight. (With the
  // next step's load skipped on some path, as a loop that tests for the
  // last step inside would have, the compiler's wait counting assumes the
  // worst and waits for every load in flight, the next step's included.)
  const int n_steps = (end > start) ? (end - start + kStep - 1) / kStep : 0;
  Tile<NU, T> A, B;
  if (n_steps > 0) {
    load_step(start, A);
    int s = 0;
    for (; s + 2 < n_steps; s += 2) {
      load_step(start + (s + 1) * kStep, B);
      compute_step(A);
      load_step(start + (s + 2) * kStep, A);
      compute_step(B);
    }
    if (s + 1 < n_steps) {
      load_step(start + (s + 1) * kStep, B);
      compute_step(A);
      compute_step(B);
    } else {
      compute_step(A);
    }
  }

  valu_wave_merge(run_m, run_l, acc);
  valu_publish(sm_acc, sm_m, sm_l, run_m, run_l, acc);
  __syncthreads();
  // merge the four waves and write the normalized partial and its LSE
  valu_finish(sm_acc, sm_m, sm_l, a.Dv, nrows - row0, [&](int gi, int d, float v, float lse) {
    const int row = row0 + gi;
    const int m = row / a.G, g = row % a.G;
    const size_t o = state_index(a, stacked, mbase, b, p, m, h * a.G + g);
    a.v_out[o * a.Dv + d] = v;
    if (d == 0) a.lse_out[o] = lse;
  });
}

}  // namespace

}  // namespace pdk
