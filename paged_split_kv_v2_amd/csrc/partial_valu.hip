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
//   * a "row group" is one DPP row of 16 lanes; it owns one token at a time,
//     lane j holding elements [j*E, (j+1)*E) of the K and V rows (E = D/16),
//     fetched with one or two 8/16-byte loads per row - a row group reads a
//     contiguous K row, a wave reads four adjacent tokens of a page;
//   * each step, the 16 row groups take 4 tokens each: token
//     t0 + u*16 + rowgroup, u = 0..3, i.e. 64 consecutive tokens;
//   * each lane keeps the running (max, sum, accumulator) of every owned
//     query row for the tokens its row group has seen (online softmax in
//     log2 units); the K/V elements it loaded are reused from registers for
//     every owned query row, so nothing is staged through LDS in the loop;
//   * q.k partial dots are summed across the row group with DPP
//     (quad_perm, row_half_mirror, row_mirror) - no LDS traffic;
//   * at the end the 16 row-group states are merged exactly (cross-row
//     shuffles inside a wave, then LDS across the 4 waves).
// With bf16 queries and keys the dot products use v_dot2_f32_bf16 (exact
// products, f32 accumulation). Values are widened to f32 (exact) and
// accumulated with f32 FMAs.

#include "device.h"
#include "internal.h"

namespace pdk {

namespace {

constexpr int kThreads = 256;
constexpr int kRowGroups = kThreads / 16;
constexpr int kTokPerRowGroup = 4;
constexpr int kStepTokens = kRowGroups * kTokPerRowGroup;  // 64

enum { KV_F32 = 0, KV_BF16 = 1 };

template <int NU>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[NU]) {
  if constexpr (NU % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NU / 4; ++i) {
      uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else if constexpr (NU == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < NU; ++i) w[i] = p[i];
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

template <int KT, int QT, int D, int GM>
__global__ __launch_bounds__(kThreads) void partial_valu_kernel(const PartialArgs a) {
  constexpr int E = D / 16;                          // elements per lane
  constexpr int NU = E * (KT == KV_F32 ? 4 : 2) / 4; // 32-bit words per lane per row
  constexpr bool kDot2 = (KT == KV_BF16 && QT == PDK_BF16);
  constexpr int QW = kDot2 ? E / 2 : E;              // per-row query registers

  __shared__ float sm_acc[4][GM][D];
  __shared__ float sm_m[4][GM];
  __shared__ float sm_l[4][GM];

  const int n_tiles = (a.max_rows + GM - 1) / GM;
  int bid = blockIdx.x;
  const int tile = bid % n_tiles;
  bid /= n_tiles;
  const int h = bid % a.Hkv;
  const int r = bid / a.Hkv;

  // request of partition row r: the largest b with part_indptr[b] <= r
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.part_indptr[mid] <= r) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int p = r - a.part_indptr[b];

  const bool stacked = a.member_indptr != nullptr;
  const int mbase = stacked ? a.member_indptr[b] : 0;
  const int nrows = (stacked ? (a.member_indptr[b + 1] - mbase) : 1) * a.G;
  const int row0 = tile * GM;
  if (row0 >= nrows) return;  // uniform over the workgroup

  const int page0 = a.indptr[b];
  const int npages = a.indptr[b + 1] - page0;
  const int start = p * a.S;
  int end = min(start + a.S, a.kv_len[b]);
  end = min(end, npages * a.P);

  const int tid = threadIdx.x;
  const int rg = tid >> 4;
  const int j = tid & 15;

  // queries of the owned rows (zero for rows past nrows)
  uint32_t qw[GM][QW];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    const int row = row0 + gi;
#pragma unroll
    for (int i = 0; i < QW; ++i) qw[gi][i] = 0;
    if (row < nrows) {
      const int m = row / a.G, g = row % a.G;
      const int qb = stacked ? a.members[mbase + m] : b;
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

  float run_m[GM], run_l[GM], acc[GM][E];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    run_m[gi] = -INFINITY;
    run_l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[gi][e] = 0.f;
  }

  const int esz = (KT == KV_F32) ? 4 : 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride * esz;
  const bool latent = a.v == nullptr;
  const char* vbase = latent ? kbase
                             : reinterpret_cast<const char*>(a.v) + (size_t)h * a.v_hstride * esz;
  const long long kb_stride = a.k_bstride * esz, vb_stride = (latent ? a.k_bstride : a.v_bstride) * esz;
  const int krow = a.Dk * esz, vrow = (latent ? a.Dk : a.Dv) * esz;

  for (int t0 = start; t0 < end; t0 += kStepTokens) {
    uint32_t kw[kTokPerRowGroup][NU], vw[kTokPerRowGroup][NU];
    bool valid[kTokPerRowGroup];
#pragma unroll
    for (int u = 0; u < kTokPerRowGroup; ++u) {
      const int t = t0 + u * 16 + rg;
      int pid = -1, slot = 0;
      if (t < end) {
        int pg;
        if (a.p_shift >= 0) { pg = t >> a.p_shift; slot = t & (a.P - 1); }
        else { pg = t / a.P; slot = t - pg * a.P; }
        pid = a.indices[page0 + pg];
      }
      valid[u] = (t < end) && (unsigned)pid < (unsigned)a.num_blocks;
      if (valid[u]) {
        load_words<NU>(reinterpret_cast<const uint32_t*>(kbase + pid * kb_stride + slot * krow) + j * NU,
                       kw[u]);
        if (latent) {
#pragma unroll
          for (int i = 0; i < NU; ++i) vw[u][i] = kw[u][i];
        } else {
          load_words<NU>(reinterpret_cast<const uint32_t*>(vbase + pid * vb_stride + slot * vrow) + j * NU,
                         vw[u]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NU; ++i) { kw[u][i] = 0; vw[u][i] = 0; }
      }
    }

    // scores s[u][gi] in log2 units
    float s[kTokPerRowGroup][GM];
#pragma unroll
    for (int u = 0; u < kTokPerRowGroup; ++u) {
      float kf[E];
      if constexpr (!kDot2) widen<KT, E, NU>(kw[u], kf);
#pragma unroll
      for (int gi = 0; gi < GM; ++gi) {
        float d = 0.f;
        if constexpr (kDot2) {
#pragma unroll
          for (int i = 0; i < QW; ++i)
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[gi][i]),
                                                __builtin_bit_cast(bf16x2_t, kw[u][i]), d, false);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) d = fmaf(bits_f32(qw[gi][e]), kf[e], d);
        }
        d = row16_sum(d);
        s[u][gi] = valid[u] ? d * a.scale_log2 : -INFINITY;
      }
    }

    float vf[kTokPerRowGroup][E];
#pragma unroll
    for (int u = 0; u < kTokPerRowGroup; ++u) widen<KT, E, NU>(vw[u], vf[u]);

#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      float mx = s[0][gi];
#pragma unroll
      for (int u = 1; u < kTokPerRowGroup; ++u) mx = fmaxf(mx, s[u][gi]);
      const float mn = fmaxf(run_m[gi], mx);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float corr = fast_exp2(run_m[gi] - mu);
      float pu[kTokPerRowGroup];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kTokPerRowGroup; ++u) {
        pu[u] = fast_exp2(s[u][gi] - mu);
        psum += pu[u];
      }
      run_l[gi] = run_l[gi] * corr + psum;
      run_m[gi] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x = acc[gi][e] * corr;
#pragma unroll
        for (int u = 0; u < kTokPerRowGroup; ++u) x = fmaf(pu[u], vf[u][e], x);
        acc[gi][e] = x;
      }
    }
  }

  // merge the four row groups of this wave (lanes l, l^16, l^32, l^48)
  const int wave = tid >> 6;
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
    if ((tid & 63) < 16) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_acc[wave][gi][j * E + e] = acc[gi][e];
      if (j == 0) {
        sm_m[wave][gi] = mw;
        sm_l[wave][gi] = l;
      }
    }
  }
  __syncthreads();

  // merge the four waves and write the normalized partial and its LSE
  for (int idx = tid; idx < GM * a.Dv; idx += kThreads) {
    const int gi = idx / a.Dv;
    const int d = idx - gi * a.Dv;
    const int row = row0 + gi;
    if (row >= nrows) continue;
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
    const int m = row / a.G, g = row % a.G;
    const int orow = (stacked ? a.out_row_base[mbase + m] : a.out_row_base[b]) + p;
    const size_t o = (size_t)orow * a.Hq + h * a.G + g;
    a.v_out[o * a.Dv + d] = (L > 0.f) ? num / L : 0.f;
    if (d == 0) a.lse_out[o] = (L > 0.f) ? M + log2f(L) : -INFINITY;
  }
}

typedef void (*KernelFn)(const PartialArgs);

template <int KT, int QT, int D>
KernelFn pick_gm(int gm) {
  constexpr int E = D / 16;
  switch (gm) {
    case 1: return partial_valu_kernel<KT, QT, D, 1>;
    case 2: return partial_valu_kernel<KT, QT, D, 2>;
    case 4: return partial_valu_kernel<KT, QT, D, 4>;
    case 8: if constexpr (8 * E <= 128) return partial_valu_kernel<KT, QT, D, 8>; else return nullptr;
    case 16: if constexpr (16 * E <= 128) return partial_valu_kernel<KT, QT, D, 16>; else return nullptr;
  }
  return nullptr;
}

template <int KT, int QT>
KernelFn pick_d(int d, int gm) {
  switch (d) {
    case 64: return pick_gm<KT, QT, 64>(gm);
    case 128: return pick_gm<KT, QT, 128>(gm);
    case 256: return pick_gm<KT, QT, 256>(gm);
  }
  return nullptr;
}

}  // namespace

// Largest query-row tile the vector path keeps in registers for head dim D.
int valu_max_rows(int D) { return D >= 256 ? 8 : 16; }

int launch_partial_valu(const PartialArgs& a, hipStream_t stream) {
  if (a.Dk != a.Dv)
    return fail(PDK_ERR_UNSUPPORTED, "vector path needs head_dim_k == head_dim_v (got %d, %d)",
                a.Dk, a.Dv);
  int gm = 1;
  while (gm < a.max_rows && gm < valu_max_rows(a.Dk)) gm <<= 1;
  KernelFn fn = nullptr;
  const int kt = a.kv_dtype, qt = a.q_dtype;
  if (kt == PDK_F32 && qt == PDK_F32) fn = pick_d<KV_F32, PDK_F32>(a.Dk, gm);
  else if (kt == PDK_F32 && qt == PDK_BF16) fn = pick_d<KV_F32, PDK_BF16>(a.Dk, gm);
  else if (kt == PDK_BF16 && qt == PDK_F32) fn = pick_d<KV_BF16, PDK_F32>(a.Dk, gm);
  else if (kt == PDK_BF16 && qt == PDK_BF16) fn = pick_d<KV_BF16, PDK_BF16>(a.Dk, gm);
  if (!fn)
    return fail(PDK_ERR_UNSUPPORTED,
                "no vector kernel for kv dtype %d, q dtype %d, head dim %d, %d rows", kt, qt,
                a.Dk, gm);
  const int n_tiles = (a.max_rows + gm - 1) / gm;
  const long long blocks = (long long)a.num_parts * a.Hkv * n_tiles;
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
