// Paged split-KV partial attention on the matrix cores (gfx950 MFMA).
//
// Used where one KV head serves at least 16 query rows: the stacked level-0
// launch of a cascade, whose rows are M members x G heads per KV head
// [cascade-PR = mlxcel pull request "perf(core): compute shared prompt
// prefixes once per decode batch", section "The decomposition, and the one
// part that is not obvious": level 0 is one request with M times as many
// query heads, so each K/V element is loaded once for all of them], and the
// 128-head latent tile of an MLA decode share [DCP-PR = ROCm/ATOM pull
// request "[feat][DCP] Optimize MLA DCP ...", section 3.2 figure: cached
// latent rows are dequantized from fp8 to bf16 and attended per chunk].
// Same contract as the vector path: one normalized partial and its log2 LSE
// per (request, partition, query row).
//
// Workgroup = NW waves, wave w owns query rows [16w, 16w+16) of the row tile.
// Per tile of TT tokens:
//   * global -> registers -> LDS, double-buffered: the next tile's loads are
//     issued in two halves, stored to the other LDS buffer after the QK
//     products and after the PV products respectively, so at most half a
//     tile of raw rows is held in registers and one barrier per tile
//     suffices. K is stored row-major [token][dim] (bf16; fp8 rows are
//     dequantized on the way: RNE_bf16(f32(x) * scale)); V transposed
//     [dim][token], written as packed token pairs;
//   * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16: A = 16 K rows from LDS,
//     B = the wave's 16 query rows (registers, loaded once). Each lane's
//     accumulator then holds one query row for four tokens;
//   * online softmax per query row in log2 units (reference maximum raised
//     lazily by > 8, as in the vector path); the row max needs two cross-lane
//     steps, the row sum is kept per lane and reduced once at the end;
//   * O^T += V^T . P^T: B = P^T straight from the S^T accumulators (the
//     MFMA's k slots of lane group q are mapped to tokens {4q..4q+3} and
//     {16+4q..16+4q+3} of each 32-token block - any permutation of the
//     contraction index is exact as long as both operands use it), A = 16
//     rows of V^T from LDS read with two 8-byte loads. P is rounded to bf16
//     and, when SPLIT, its remainder is rounded and accumulated by a second
//     MFMA (p = hi + lo to about 16 bits), so the partial stays within f32-
//     level error of the vector path.
// All products of bf16 inputs are exact in the f32 accumulators.

#include "device.h"
#include "internal.h"
#include "rows.h"

namespace pdk {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum { MK_BF16 = 1, MK_FP8 = 2 };
constexpr int kMaxPartPagesM = 1024;
constexpr float kLazyLog2M = 8.f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ u32x4_t ld_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Pair word of element e from two rows of packed bf16: low half from row 0.
__device__ __forceinline__ uint32_t pair_word(const uint32_t* w0, const uint32_t* w1, int e) {
  const uint32_t a = w0[e >> 1], b = w1[e >> 1];
  return (e & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
}

template <int DK, int DV, int NW, int TT, int KT, bool LATENT, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void partial_mfma_kernel(const PartialArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int KSTEPS = DK / 32;
  constexpr int TB = TT / 16;                    // 16-token blocks per tile
  constexpr int KB = TT / 32;                    // 32-token contraction blocks per tile
  constexpr int DB = DV / 16;                    // 16-wide output column blocks
  constexpr int KLD = DK + 8;                    // LDS row of K (bf16), padded 16 B
  constexpr int VLD = TT + 4;                    // LDS row of V^T (bf16), padded 8 B
  constexpr int KCW = (KT == MK_FP8) ? 16 : 8;   // elements per 16-byte chunk
  constexpr int KCH = DK / KCW;                  // chunks per K row
  constexpr int VCH = DV / KCW;                  // chunks per V row
  constexpr int KPAIRS = (TT / 2) * KCH;         // (token pair, chunk) items of K per tile
  constexpr int VPAIRS = LATENT ? 0 : (TT / 2) * VCH;
  constexpr int ITEMS = KPAIRS + VPAIRS;
  constexpr int NIT = (ITEMS + NT - 1) / NT;     // items per thread per tile
  constexpr int NA = (NIT + 1) / 2;              // first half: staged after the QK products
  constexpr int KW = KCW / 2;                    // bf16 words of a converted chunk
  static_assert(DK % 32 == 0 && DV % 16 == 0 && TT % 32 == 0, "tile shapes");
  static_assert(!LATENT || (DV <= DK && DV % KCW == 0), "latent value lanes");

  // two LDS buffers: the next tile is staged while the current one is read
  __shared__ __align__(16) uint16_t sm_k[2][TT * KLD];
  __shared__ __align__(16) uint16_t sm_vt[2][DV * VLD];
  __shared__ int sm_pid[kMaxPartPagesM];

  const int n_tiles = (a.max_rows + 16 * NW - 1) / (16 * NW);
  int unit, tile;
  xcd_unit_tile(blockIdx.x, n_tiles, unit, tile);
  if (unit >= a.num_parts * a.Hkv) return;  // grid padding (uniform)
  const int h = unit % a.Hkv;
  const int r = unit / a.Hkv;
  const int tid = threadIdx.x;

  int b = 0, p;
  if (a.work != nullptr) {
    const int2 it = a.work[r];
    b = it.x;
    p = it.y;
  } else {
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
  const int row0 = tile * 16 * NW;
  if (row0 >= nrows) return;  // uniform

  int page0, start, end;
  part_range(a, b, p, page0, start, end);
  // causal rows: the tile loop stops at the last owned row's end
  end = min(end, visible_end(a, b, (min(row0 + 16 * NW, nrows) - 1) / a.G));
  const int shift = a.p_shift;
  const int pmask = a.P - 1;
  const int pg_first = start >> shift;
  if (end > start) {
    const int n_pg = ((end - 1) >> shift) - pg_first + 1;
    for (int i = tid; i < n_pg; i += NT) {
      const int pid = a.indices[page0 + pg_first + i];
      // an id outside the pool reads row 0 (see part_range)
      sm_pid[i] = ((unsigned)pid < (unsigned)a.num_blocks) ? pid : 0;
    }
  }

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int q4 = lane >> 4;   // lane group
  const int r16 = lane & 15;  // query row within the wave / MFMA column

  // the wave's 16 query rows as MFMA B fragments (bf16)
  u32x4_t qf[KSTEPS];
  const int my_row = row0 + 16 * wave + r16;
  // positions this lane's row sees within the partition
  const int my_end = min(end, visible_end(a, b, min(my_row, nrows - 1) / a.G));
  {
    int qb = b, head = 0;
    const bool live = my_row < nrows;
    if (live) {
      const int m = my_row / a.G, g = my_row % a.G;
      qb = query_row(a, stacked, mbase, b, m);
      head = h * a.G + g;
    }
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qb * a.Hq + head) * DK;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = live ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks + 8 * q4)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  constexpr int ESZ = (KT == MK_FP8) ? 1 : 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride * ESZ;
  const char* vbase = LATENT ? kbase
                             : reinterpret_cast<const char*>(a.v) + (size_t)h * a.v_hstride * ESZ;
  const long long kb_stride = a.k_bstride * ESZ;
  const long long vb_stride = (LATENT ? a.k_bstride : a.v_bstride) * ESZ;
  const int krow = DK * ESZ, vrow = (LATENT ? DK : DV) * ESZ;

  u32x4_t raw[NIT][2];  // staged items: two tokens of one 16-byte chunk each

  auto row_addr = [&](const char* base, long long bstride, int rowb, int t) {
    const int tc = min(t, end - 1);
    const int pid = sm_pid[(tc >> shift) - pg_first];
    return base + pid * bstride + (tc & pmask) * rowb;
  };
  // item c < KPAIRS: K chunk (token pair c / KCH, chunk c % KCH); else V
  auto is_k = [&](int it, int c) {
    if constexpr (KPAIRS % NT == 0) return it < KPAIRS / NT;
    else return c < KPAIRS;
  };

  auto load_items = [&](int it0, int it1, int t0) {
#pragma unroll
    for (int it = it0; it < it1; ++it) {
      const int c = tid + it * NT;
      if (ITEMS % NT == 0 || c < ITEMS) {
        if (is_k(it, c)) {
          const int tp = c / KCH, cc = c - tp * KCH;
#pragma unroll
          for (int s = 0; s < 2; ++s)
            raw[it][s] = ld_nt16(row_addr(kbase, kb_stride, krow, t0 + 2 * tp + s) + cc * 16);
        } else {
          const int c2 = c - KPAIRS;
          const int tp = c2 / VCH, vc = c2 - tp * VCH;
#pragma unroll
          for (int s = 0; s < 2; ++s)
            raw[it][s] = ld_nt16(row_addr(vbase, vb_stride, vrow, t0 + 2 * tp + s) + vc * 16);
        }
      }
    }
  };

  // 16 bytes of stored K/V -> packed bf16 words (fp8: 16 values -> 8 words)
  auto convert = [&](const u32x4_t& x, uint32_t* w, float scale) {
    if constexpr (KT == MK_FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fp8x4_dequant_bf16(x[i], scale, w[2 * i], w[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = x[i];
    }
  };

  auto store_items = [&](int it0, int it1, int bf) {
#pragma unroll
    for (int it = it0; it < it1; ++it) {
      const int c = tid + it * NT;
      if (ITEMS % NT == 0 || c < ITEMS) {
        if (is_k(it, c)) {
          const int tp = c / KCH, cc = c - tp * KCH;
          const bool vt = LATENT && cc * KCW < DV;  // these lanes are also values
          if constexpr (KT == MK_FP8) {
            // four codes of each token at a time: 8-byte K pieces, 4 V^T pairs
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t w0[2], w1[2];
              fp8x4_dequant_bf16(raw[it][0][i], a.k_scale, w0[0], w0[1]);
              fp8x4_dequant_bf16(raw[it][1][i], a.k_scale, w1[0], w1[1]);
              *reinterpret_cast<u32x2_t*>(&sm_k[bf][(2 * tp) * KLD + cc * KCW + 4 * i]) =
                  u32x2_t{w0[0], w0[1]};
              *reinterpret_cast<u32x2_t*>(&sm_k[bf][(2 * tp + 1) * KLD + cc * KCW + 4 * i]) =
                  u32x2_t{w1[0], w1[1]};
              if (vt) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  *reinterpret_cast<uint32_t*>(&sm_vt[bf][(cc * KCW + 4 * i + e) * VLD + 2 * tp]) =
                      pair_word(w0, w1, e);
              }
            }
          } else {
            uint32_t w[2][KW];
            convert(raw[it][0], w[0], a.k_scale);
            convert(raw[it][1], w[1], a.k_scale);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
              for (int i = 0; i < KW / 4; ++i)
                *reinterpret_cast<u32x4_t*>(&sm_k[bf][(2 * tp + s) * KLD + cc * KCW + 8 * i]) =
                    u32x4_t{w[s][4 * i], w[s][4 * i + 1], w[s][4 * i + 2], w[s][4 * i + 3]};
            if (vt) {
#pragma unroll
              for (int e = 0; e < KCW; ++e)
                *reinterpret_cast<uint32_t*>(&sm_vt[bf][(cc * KCW + e) * VLD + 2 * tp]) =
                    pair_word(w[0], w[1], e);
            }
          }
        } else {
          uint32_t w[2][KW];
          const int c2 = c - KPAIRS;
          const int tp = c2 / VCH, vc = c2 - tp * VCH;
          convert(raw[it][0], w[0], a.v_scale);
          convert(raw[it][1], w[1], a.v_scale);
#pragma unroll
          for (int e = 0; e < KCW; ++e)
            *reinterpret_cast<uint32_t*>(&sm_vt[bf][(vc * KCW + e) * VLD + 2 * tp]) =
                pair_word(w[0], w[1], e);
        }
      }
    }
  };

  f32x4_t acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float run_m = -INFINITY, run_l = 0.f;

  __syncthreads();  // page ids visible
  if (start < end) {
    load_items(0, NIT, start);
    store_items(0, NIT, 0);
  }
  __syncthreads();
  int bf = 0;
  for (int t0 = start; t0 < end; t0 += TT) {
    const bool more = t0 + TT < end;  // uniform
    if (more) load_items(0, NA, t0 + TT);

    // S^T = K . Q^T for the wave's 16 query rows
    f32x4_t s[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      s[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(
            &sm_k[bf][(16 * tb + r16) * KLD + 32 * ks + 8 * q4]);
        s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), s[tb],
                                                        0, 0, 0);
      }
    }
    if (more) {
      store_items(0, NA, bf ^ 1);
      load_items(NA, NIT, t0 + TT);
    }

    // scale, mask tokens past the end, row max across the four lane groups
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 16 * tb + 4 * q4 + j;
        s[tb][j] = (t < my_end) ? s[tb][j] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[tb][j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int need = mx > run_m + kLazyLog2M;
    if (__any(need)) {
      const float mn = need ? mx : run_m;
      const float corr = (mn == run_m) ? 1.f : fast_exp2(run_m - mn);
      run_l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= corr;
      run_m = mn;
    }
    const float mu = (run_m == -INFINITY) ? 0.f : run_m;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[tb][j] = fast_exp2(s[tb][j] - mu);
        run_l += s[tb][j];
      }

    // O^T += V^T . P^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4_t& sv = s[2 * kb + i];
        hw[2 * i] = pack_bf16x2_rne(sv[0], sv[1]);
        hw[2 * i + 1] = pack_bf16x2_rne(sv[2], sv[3]);
        if constexpr (SPLIT) {
          lw[2 * i] = pack_bf16x2_rne(sv[0] - bf16_lo(hw[2 * i]), sv[1] - bf16_hi(hw[2 * i]));
          lw[2 * i + 1] =
              pack_bf16x2_rne(sv[2] - bf16_lo(hw[2 * i + 1]), sv[3] - bf16_hi(hw[2 * i + 1]));
        }
      }
      const bf16x8_t ph = as_bf16x8(u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      bf16x8_t pl;
      if constexpr (SPLIT) pl = as_bf16x8(u32x4_t{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vp = &sm_vt[bf][(16 * db + r16) * VLD + 32 * kb + 4 * q4];
        const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(vp);
        const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(vp + 16);
        const bf16x8_t vf = as_bf16x8(u32x4_t{v0[0], v0[1], v1[0], v1[1]});
        acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph, acc_o[db], 0, 0, 0);
        if constexpr (SPLIT)
          acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, acc_o[db], 0, 0, 0);
      }
    }
    if (more) store_items(NA, NIT, bf ^ 1);
    __syncthreads();  // next tile staged; this tile's buffer free again
    bf ^= 1;
  }

  // row sum across the lane groups, then the normalized partial and its LSE
  float l = run_l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (my_row < nrows) {
    const int m = my_row / a.G, g = my_row % a.G;
    const size_t o = state_index(a, stacked, mbase, b, p, m, h * a.G + g);
    float* dst = a.v_out + o * DV + 4 * q4;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (l > 0.f) x = make_float4(acc_o[db][0] / l, acc_o[db][1] / l, acc_o[db][2] / l, acc_o[db][3] / l);
      *reinterpret_cast<float4*>(dst + 16 * db) = x;
    }
    if (q4 == 0) a.lse_out[o] = (l > 0.f) ? run_m + log2f(l) : -INFINITY;
  }
}

typedef void (*MfmaFn)(const PartialArgs);

}  // namespace

// Partial launch on the matrix cores when an instantiation covers the shape:
// more than 16 bf16 query rows per KV head (one tile of 32 or 64 rows, or
// several tiles), head dims 128/128 with bf16 K and V, or the 576/512 latent
// tile with bf16 or fp8 rows and at least 64 query rows.
int launch_partial_mfma(const PartialArgs& a, hipStream_t stream, bool* handled) {
  *handled = false;
  if (a.q_dtype != PDK_BF16 || a.max_rows <= 16 || a.p_shift < 0) return PDK_OK;
  MfmaFn fn = nullptr;
  int nw = 0;
  const bool latent = a.v == nullptr;
  if (a.Dk == 128 && a.Dv == 128 && !latent && a.kv_dtype == PDK_BF16 && a.max_rows > 16) {
    nw = a.max_rows <= 32 ? 2 : 4;
    fn = nw == 2 ? partial_mfma_kernel<128, 128, 2, 64, MK_BF16, false, true>
                 : partial_mfma_kernel<128, 128, 4, 64, MK_BF16, false, true>;
  } else if (a.Dk == 576 && a.Dv == 512 && latent && a.max_rows >= 64) {
    nw = 8;
    fn = a.kv_dtype == PDK_FP8_E4M3 ? partial_mfma_kernel<576, 512, 8, 32, MK_FP8, true, false>
       : a.kv_dtype == PDK_BF16     ? partial_mfma_kernel<576, 512, 8, 32, MK_BF16, true, true>
                                    : nullptr;
  }
  if (!fn) return PDK_OK;
  if (a.S / a.P + 1 > kMaxPartPagesM)
    return fail(PDK_ERR_UNSUPPORTED, "partition of %d tokens spans more than %d pages", a.S,
                kMaxPartPagesM - 1);
  *handled = true;
  const int n_tiles = (a.max_rows + 16 * nw - 1) / (16 * nw);
  const long long blocks = xcd_grid_blocks((long long)a.num_parts * a.Hkv, n_tiles);
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * nw), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "mfma partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
