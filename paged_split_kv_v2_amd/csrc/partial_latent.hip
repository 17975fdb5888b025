// Paged split-KV partial attention for a latent (MLA) pool on the matrix
// cores: 576-wide latent rows, values = their first 512 lanes, one KV head
// serving 128 query heads [DCP-PR = ROCm/ATOM pull request "[feat][DCP]
// Optimize MLA DCP ...", section 3.2 figure: cached latent rows are
// dequantized from fp8 to bf16 and attended chunk by chunk, each chunk
// returning its output and LSE; section 3.3: per-tensor fp8 scale]. Same
// contract as the other partial kernels: one normalized partial and its log2
// LSE per (request, partition, query row).
//
// Workgroup = 4 waves, 64 query rows; two workgroups share a CU (two waves
// per SIMD), so one computes while the other waits at a barrier or on LDS.
// Waves w and w^2 share rows [32(w%2), 32(w%2)+32) for the whole partition
// and split the work on them in halves:
//   * S^T: wave half hf contracts the 16-dim k-steps 2ks + hf (ks < 18) with
//     its half of Q^T held as B operands of v_mfma_f32_32x32x16_bf16 (18
//     k-steps x 8 bf16 per lane); the two partial sums are exchanged through
//     LDS and added, so both waves hold the same S^T (IEEE addition
//     commutes);
//   * O^T: wave half hf accumulates value dims [256hf, 256hf+256) as 8
//     accumulator blocks of 32x32 (128 registers per lane);
//   * the tile (32 tokens) is staged in LDS as bf16 [token][576] (fp8 rows
//     dequantized on the way: RNE_bf16(f32(x) * scale)); 16-byte chunks are
//     XOR-swizzled by token so that both reads below are free of bank
//     conflicts;
//   * S^T = K . Q^T: A = 32 K rows read with 16-byte loads;
//   * O^T += V^T . P^T: A = 32 value dims x 16 tokens read straight from the
//     row-major tile with the gfx950 transposing LDS load (ds_read_b64_tr_b16:
//     in each group of 16 lanes, lane i receives element i%4 of the 8 bytes
//     addressed by lane 4e + i/4 as its element e), no transposed copy; B =
//     P^T taken from the S^T accumulators as they lie (the MFMA's k slots of
//     lane half h are the tokens {4h..4h+3, 8+4h..8+4h+3} of each 16-token
//     block, and the V^T loads use the same token order);
//   * online softmax per query row in log2 units, lazy reference maximum as
//     in the other kernels; P is rounded to bf16 for the PV product.
// The next tile's rows are fetched with gfx950's global->LDS loads (16 bytes
// per lane, placed at base + 16*lane) into a raw staging buffer before the
// products of the current tile; after them each lane converts the 16 bytes
// it fetched itself into the tile buffer, so no registers hold rows in
// flight. Three barriers per tile: S^T exchange, tile buffer free, tile
// buffer filled. The two row halves of a partition are issued 8 blocks apart,
// which lands them on the same XCD (blocks are dealt round-robin to the 8
// XCDs) at about the same time: the second reads the rows from that L2.

#include "device.h"
#include "internal.h"

namespace pdk {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

enum { LK_BF16 = 1, LK_FP8 = 2 };
constexpr int kTT = 32;          // tokens per tile
constexpr int kWaves = 4;
constexpr int kRows = 64;
constexpr int kMaxPagesL = 256;  // pages of one partition (plus one)
constexpr float kLazyL = 8.f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ u32x4_t ld_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Stored position of 16-byte chunk q of token row t. The swizzle permutes
// chunks within aligned groups of 8: rows of equal parity get distinct
// positions for 16 consecutive tokens (16-byte loads of one chunk), and rows
// t and t+2 of an aligned group of 4 land in different halves of the group
// (8-byte transposing loads of 4 tokens x 4 chunks).
__device__ __forceinline__ int swz(int t, int q) { return q ^ ((5 * (t >> 1)) & 7); }

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its global->LDS fetches still in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
enum : int { SG_MFMA = 0x008, SG_DS_READ = 0x100 };

template <int DK, int DV, int KT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void partial_latent_kernel(const PartialArgs a) {
  constexpr int NT = 64 * kWaves;
  constexpr int KS = DK / 32;                       // k-steps of S^T per contraction half
  constexpr int DB = DV / 64;                       // 32-dim output blocks per value half
  constexpr int ESZ = (KT == LK_FP8) ? 1 : 2;
  constexpr int RCH = DK * ESZ / 16;                // 16-byte stored chunks per token
  constexpr int ITEMS = kTT * RCH;
  constexpr int NBLK = ITEMS / 64;                  // 64-item blocks (one per wave load)
  static_assert(ITEMS % 64 == 0, "whole blocks");
  static_assert(DK % 64 == 0 && DV % 32 == 0 && DV <= DK, "latent shapes");

  __shared__ __align__(16) uint16_t sk[kTT * DK];
  __shared__ __align__(16) u32x4_t sraw[ITEMS];         // fetched rows, item order
  __shared__ __align__(16) u32x4_t xs[kWaves][4][64];  // partial S^T of each wave
  __shared__ int sm_pid[kMaxPagesL];

  // block -> (unit = partition * Hkv + kv head, row tile): the row tiles of a
  // unit are 8 blocks apart, 8 units per group
  const int n_tiles = (a.max_rows + kRows - 1) / kRows;
  const int bid = blockIdx.x;
  const int unit = 8 * (bid / (8 * n_tiles)) + (bid & 7);
  const int tile = (bid >> 3) % n_tiles;
  if (unit >= a.num_parts * a.Hkv) return;  // uniform: padding of the last group
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
  const int nrows = (stacked ? (a.member_indptr[b + 1] - mbase) : 1) * a.G;
  const int row0 = tile * kRows;
  if (row0 >= nrows) return;  // uniform

  const int page0 = a.indptr[b];
  const int npages = a.indptr[b + 1] - page0;
  const int start = p * a.S;
  int end = min(start + a.S, a.kv_len[b]);
  end = min(end, npages * a.P);
  const int shift = a.p_shift;
  const int pmask = a.P - 1;
  const int pg_first = start >> shift;
  if (end > start) {
    const int n_pg = ((end - 1) >> shift) - pg_first + 1;
    for (int i = tid; i < n_pg; i += NT) {
      const int pid = a.indices[page0 + pg_first + i];
      // an id outside the pool reads row 0: wrong numbers, never a fault
      sm_pid[i] = ((unsigned)pid < (unsigned)a.num_blocks) ? pid : 0;
    }
  }

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;   // lane half
  const int c32 = lane & 31;  // MFMA column (query row) / A row
  const int hf = wave >> 1;   // contraction half of S^T, value half of O^T

  // half of the 32 query rows as B fragments: lane -> row c32,
  // dims 16(2ks + hf) + 8hl + i
  u32x4_t qf[KS];
  const int my_row = row0 + 32 * (wave & 1) + c32;
  {
    int qb = b, head = 0;
    const bool live = my_row < nrows;
    if (live) {
      const int m = my_row / a.G, g = my_row % a.G;
      qb = stacked ? a.members[mbase + m] : b;
      head = h * a.G + g;
    }
    // row 0 of request qb stands in for padding rows: always a valid address
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)qb * a.Hq + head) * DK + 16 * hf + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
      qf[ks] = live ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride * ESZ;
  const long long kb_stride = a.k_bstride * ESZ;
  constexpr int krow = DK * ESZ;

  // Item c of a tile: token c / RCH, stored 16-byte chunk c % RCH. Block k
  // (items 64k..64k+63) is fetched and later converted by wave k % kWaves,
  // lane i handling item 64k + i.
  // A tile never crosses a page (P is a multiple of the tile), so one page
  // id serves all its rows; rows past the end repeat the last token.
  auto fetch_tile = [&](int t0) {
    const int pid = __builtin_amdgcn_readfirstlane(sm_pid[(t0 >> shift) - pg_first]);
    const char* pbase = kbase + pid * kb_stride + (long long)(t0 & pmask) * krow;
    const int tlim = end - 1 - t0;
    for (int k = wave; k < NBLK; k += kWaves) {
      const int c = 64 * k + lane;
      const int tt = c / RCH, rc = c - tt * RCH;
      __builtin_amdgcn_global_load_lds(pbase + min(tt, tlim) * krow + rc * 16,
                                       (__attribute__((address_space(3))) void*)&sraw[64 * k],
                                       16, 0, 0);
    }
  };
  auto convert_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fetches have landed
    for (int k = wave; k < NBLK; k += kWaves) {
      const int c = 64 * k + lane;
      const int tt = c / RCH, rc = c - tt * RCH;
      const u32x4_t x = sraw[c];
      uint16_t* row = &sk[tt * DK];
      if constexpr (KT == LK_FP8) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {  // 8 codes -> one 16-byte bf16 chunk
          uint32_t w[4];
          fp8x4_dequant_bf16(x[2 * hh], a.k_scale, w[0], w[1]);
          fp8x4_dequant_bf16(x[2 * hh + 1], a.k_scale, w[2], w[3]);
          *reinterpret_cast<u32x4_t*>(row + 8 * swz(tt, 2 * rc + hh)) = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      } else {
        *reinterpret_cast<u32x4_t*>(row + 8 * swz(tt, rc)) = x;
      }
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  float run_m = -INFINITY, run_l = 0.f;

  // Per-lane LDS element offsets within a tile buffer. The swizzle only
  // permutes the low three bits of the chunk index, so each read below is a
  // per-lane base plus a compile-time offset:
  //   K fragment of k-step 2ks + hf: row c32, chunk 4ks + 2hf + hl
  //     -> c32*DK + 64(ks/2) + 8((2hf + hl) ^ f(c32) ^ 4(ks%2));
  //   V^T fragment (kb, rho, db): token 16kb + 8rho + tr_tok, dims
  //     (DV/2)hf + 32db + tr_dim -> chunk 32hf + 4db + e with e = tr_dim/8,
  //     swizzled by f(t) = y ^ 4rho, y = 5(tr_tok/2) mod 8.
  const int fk = (5 * (c32 >> 1)) & 7;
  const int kofs0 = c32 * DK + 8 * ((2 * hf + hl) ^ fk);
  const int kofs1 = c32 * DK + 8 * ((2 * hf + hl) ^ fk ^ 4);
  const int tr_tok = 4 * hl + ((lane & 15) >> 2);
  const int tr_e = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_z = tr_e ^ ((5 * (tr_tok >> 1)) & 7);
  const int vbase = tr_tok * DK + (DV / 2) * hf + 4 * (lane & 1);
  const int vofs0 = vbase + 8 * tr_z;
  const int vofs1 = vbase + 8 * (tr_z ^ 4);

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query fragments have landed
  __syncthreads();                     // page ids visible
  if (start < end) {
    fetch_tile(start);
    convert_tile();
  }
  __syncthreads();
  for (int t0 = start; t0 < end; t0 += kTT) {
    const bool more = t0 + kTT < end;  // uniform
    const uint16_t* tile_k = sk;

    // S^T = K . Q^T: lane -> query row c32, tokens 8(j/4) + 4hl + j%4
    f32x16_t s;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = 0.f;
    {
      // K fragments are read KP k-steps ahead of their product
      constexpr int KP = 2;
      u32x4_t kf[KS];
      auto kread = [&](int ks) {
        return *reinterpret_cast<const u32x4_t*>(tile_k + ((ks & 1) ? kofs1 : kofs0) +
                                                 64 * (ks >> 1));
      };
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) kf[ks] = kread(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + KP < KS) kf[ks + KP] = kread(ks + KP);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks]), as_bf16x8(qf[ks]), s, 0,
                                                    0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, KP, 0);
#pragma unroll
      for (int i = 0; i < KS - KP; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, KP, 0);
    }
    if (more) fetch_tile(t0 + kTT);
    // exchange the partial sums with the other half
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xs[wave][q][lane] = u32x4_t{f32_bits(s[4 * q]), f32_bits(s[4 * q + 1]),
                                  f32_bits(s[4 * q + 2]), f32_bits(s[4 * q + 3])};
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t o = xs[wave ^ 2][q][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * q + i] += bits_f32(o[i]);
    }

    // row max over the two lane halves, in scaled log2 units; a full tile
    // scales inside the exponent below, the last tile masks first
    float cs = a.scale_log2, mx;
    if (t0 + kTT <= end) {
      float hi = fmaxf(s[0], s[1]), lo = fminf(s[0], s[1]);
#pragma unroll
      for (int j = 2; j < 16; j += 2) {
        hi = fmaxf(hi, fmaxf(s[j], s[j + 1]));
        lo = fminf(lo, fminf(s[j], s[j + 1]));
      }
      mx = (cs >= 0.f ? hi : lo) * cs;
    } else {
      mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + 8 * (j >> 2) + 4 * hl + (j & 3);
        s[j] = (t < end) ? s[j] * cs : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      cs = 1.f;
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(f32_bits(mx), f32_bits(mx), false, false);
      mx = fmaxf(bits_f32(sw[0]), bits_f32(sw[1]));  // max over lanes l and l ^ 32
    }
    const int need = mx > run_m + kLazyL;
    if (__any(need)) {
      const float mn = need ? mx : run_m;
      const float corr = (mn == run_m) ? 1.f : fast_exp2(run_m - mn);
      run_l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= corr;
      run_m = mn;
    }
    const float mu = (run_m == -INFINITY) ? 0.f : run_m;
    uint32_t pw[8];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[j], cs, -mu));
      const float p1 = fast_exp2(__builtin_fmaf(s[j + 1], cs, -mu));
      run_l += p0 + p1;
      pw[j >> 1] = pack_bf16x2_rne(p0, p1);
    }
    const bf16x8_t pb0 = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8_t pb1 = as_bf16x8(u32x4_t{pw[4], pw[5], pw[6], pw[7]});

    // O^T += V^T . P^T, V^T fragments by transposing loads issued VP
    // products ahead; step i = (db, kb) = (i / 2, i % 2)
    {
      constexpr int NS = 2 * DB, VP = 1;
      u32x4_t vf[NS];
      auto vread = [&](int i) {
        const int db = i >> 1, kb = i & 1;
        s16x4_t v[2];
#pragma unroll
        for (int rho = 0; rho < 2; ++rho) {
          const uint16_t* ptr = tile_k + (((db & 1) ^ rho) ? vofs1 : vofs0) +
                                (16 * kb + 8 * rho) * DK + 64 * (db >> 1);
          v[rho] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)ptr);
        }
        const u32x2_t v0 = __builtin_bit_cast(u32x2_t, v[0]), v1 = __builtin_bit_cast(u32x2_t, v[1]);
        return u32x4_t{v0[0], v0[1], v1[0], v1[1]};
      };
#pragma unroll
      for (int i = 0; i < VP; ++i) vf[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + VP < NS) vf[i + VP] = vread(i + VP);
        acc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[i]), (i & 1) ? pb1 : pb0,
                                                              acc[i >> 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * VP, 0);
#pragma unroll
      for (int i = 0; i < NS - VP; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, VP, 0);
    }
    if (more) {
      lds_barrier();  // every wave is done with the tile buffer
      convert_tile();
    }
    lds_barrier();  // next tile staged; exchange slots free again
  }

  // row sum over the lane halves, normalized partial and its LSE
  float l = run_l;
  l += __shfl_xor(l, 32);
  if (my_row < nrows) {
    const int m = my_row / a.G, g = my_row % a.G;
    const int orow = (stacked ? a.out_row_base[mbase + m] : a.out_row_base[b]) + p;
    const size_t o = (size_t)orow * a.Hq + h * a.G + g;
    float* dst = a.v_out + o * DV + (DV / 2) * hf + 4 * hl;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        *reinterpret_cast<float4*>(dst + 32 * db + 8 * jb) =
            make_float4(acc[db][4 * jb] * inv, acc[db][4 * jb + 1] * inv,
                        acc[db][4 * jb + 2] * inv, acc[db][4 * jb + 3] * inv);
    if (hl == 0 && hf == 0) a.lse_out[o] = (l > 0.f) ? run_m + log2f(l) : -INFINITY;
  }
}

typedef void (*LatentFn)(const PartialArgs);

}  // namespace

// Latent pools (values = the first Dv lanes of each 576-wide key row, one
// KV head) with bf16 queries, fp8 or bf16 rows, at least 64 query rows per
// KV head and pages of a multiple of 32 tokens; *handled says whether this
// path took the launch.
int launch_partial_latent(const PartialArgs& a, hipStream_t stream, bool* handled) {
  *handled = false;
  if (a.q_dtype != PDK_BF16 || a.v != nullptr || a.Dk != 576 || a.Dv != 512 ||
      a.max_rows < 64 || a.p_shift < 0 || a.P % kTT != 0)
    return PDK_OK;
  LatentFn fn = a.kv_dtype == PDK_FP8_E4M3 ? partial_latent_kernel<576, 512, LK_FP8>
              : a.kv_dtype == PDK_BF16     ? partial_latent_kernel<576, 512, LK_BF16>
                                           : nullptr;
  if (!fn) return PDK_OK;
  if (a.S / a.P + 1 > kMaxPagesL)
    return fail(PDK_ERR_UNSUPPORTED, "partition of %d tokens spans more than %d pages", a.S,
                kMaxPagesL - 1);
  *handled = true;
  const int n_tiles = (a.max_rows + kRows - 1) / kRows;
  const long long units = (long long)a.num_parts * a.Hkv;
  const long long blocks = (units + 7) / 8 * 8 * n_tiles;
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "latent partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
