// Paged split-KV partial attention for a latent (MLA) pool on the matrix
// cores: 576-wide latent rows, values = their first 512 lanes, one KV head
// serving 128 query heads [DCP-PR = ROCm/ATOM pull request "[feat][DCP]
// Optimize MLA DCP ...", section 3.2 figure: cached latent rows are
// dequantized from fp8 to bf16 and attended chunk by chunk, each chunk
// returning its output and LSE; section 3.3: per-tensor fp8 scale]. Same
// contract as the other partial kernels: one normalized partial and its log2
// LSE per (request, partition, query row).
//
// Workgroup = 8 waves (two per SIMD), 128 query rows, or 4 waves and 64
// rows for launches whose 128-row grid would not cover the CUs (a short new-
// token range split into few partitions); wave w owns rows [16w, 16w+16)
// for the whole partition:
//   * Q^T as B operands of v_mfma_f32_16x16x32_bf16 (18 k-steps x 8 bf16 per
//     lane) and O^T = 512 dims x 16 rows as 32 accumulator blocks of 16x16
//     (128 registers per lane); no exchange between waves;
//   * the tile (32 tokens) is staged in LDS as bf16 [token][576] (fp8 rows
//     dequantized on the way: RNE_bf16(f32(x) * scale)); 16-byte chunks are
//     XOR-swizzled by token so that both reads below are free of bank
//     conflicts;
//   * S^T = K . Q^T: A = 16 K rows read with 16-byte loads (two 16-token
//     blocks per tile);
//   * O^T += V^T . P^T: A = 16 value dims x 32 tokens read straight from the
//     row-major tile with the gfx950 transposing LDS load (ds_read_b64_tr_b16:
//     in each group of 16 lanes, lane i receives element i%4 of the 8 bytes
//     addressed by lane 4e + i/4 as its element e), no transposed copy; B =
//     P^T taken from the S^T accumulators as they lie (the MFMA's k slots of
//     lane group q are the tokens {4q..4q+3} and {16+4q..16+4q+3}, and the V^T
//     loads use the same token order);
//   * online softmax per query row in log2 units, lazy reference maximum as
//     in the other kernels; P enters the PV product as bf16 hi + lo parts
//     (two products per block).
// Pipeline: three bf16 tile buffers and one raw staging buffer. While tile i
// is multiplied from one buffer, tile i + 1 (fetched during tile i - 1 by
// gfx950's global->LDS loads, 16 bytes per lane at base + 16*lane) is
// dequantized into another by the waves that fetched its bytes (8 codes per
// lane, consecutive lanes writing consecutive chunks: no bank conflicts),
// and tile i + 2 is then fetched; one barrier per tile. The second half of
// the waves applies each tile's PV product one tile late, so that on each
// SIMD one wave's softmax and dequantization run beside the other wave's
// products. No registers hold rows in flight. (Measured on 32 requests x
// 16K fp8 tokens: 211 -> 204 us per launch; the conflict-free
// dequantization alone removes a quarter of the LDS bank-conflict cycles
// but does not change the time.)

#include "device.h"
#include "internal.h"
#include "rows.h"

namespace pdk {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

enum { LK_BF16 = 1, LK_FP8 = 2 };
constexpr int kTT = 32;          // tokens per tile
constexpr int kMaxPagesL = 256;  // pages of one partition (plus one)
constexpr int kChipCUs = 256;    // compute units of an MI355X
constexpr float kLazyL = 8.f;
constexpr bool kStagger = true;  // second half of the waves one PV product behind

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

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

template <int DK, int DV, int KT, int kWaves>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void partial_latent_kernel(const PartialArgs a) {
  constexpr int kRows = 16 * kWaves;  // query rows per workgroup
  constexpr int NT = 64 * kWaves;
  constexpr int KS = DK / 32;                       // k-steps of S^T (32 dims)
  constexpr int DB = DV / 16;                       // 16-dim output blocks
  constexpr int ESZ = (KT == LK_FP8) ? 1 : 2;
  constexpr int RCH = DK * ESZ / 16;                // 16-byte stored chunks per token
  constexpr int ITEMS = kTT * RCH;
  constexpr int NBLK = ITEMS / 64;                  // 64-item blocks (one per wave load)
  static_assert(ITEMS % 64 == 0, "whole blocks");
  static_assert(DK % 64 == 0 && DV % 32 == 0 && DV <= DK, "latent shapes");

  // three bf16 tile buffers and one raw staging buffer, each its own LDS
  // object: the compiler tells accesses of distinct objects apart from the
  // global->LDS loads in flight, and otherwise waits for those loads
  __shared__ __align__(16) uint16_t sk0[kTT * DK];
  __shared__ __align__(16) uint16_t sk1[kTT * DK];
  __shared__ __align__(16) uint16_t sk2[kTT * DK];
  __shared__ __align__(16) u32x4_t sraw[ITEMS];  // fetched rows, item order
  __shared__ int sm_pid[kMaxPagesL];

  // block -> (unit = partition * Hkv + kv head, row tile), a unit's row
  // tiles on one XCD
  const int n_tiles = (a.max_rows + kRows - 1) / kRows;
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
  const int row0 = tile * kRows;
  if (row0 >= nrows) return;  // uniform

  int page0, start, end;
  part_range(a, b, p, page0, start, end);
  // causal rows: the tile loop stops at the last owned row's end; every
  // owned row sees at least the positions below end_lo (uniform)
  const int end_lo = min(end, visible_end(a, b, row0 / a.G));
  end = min(end, visible_end(a, b, (min(row0 + kRows, nrows) - 1) / a.G));
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

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int q4 = lane >> 4;   // lane group
  const int r16 = lane & 15;  // query row of the wave / MFMA column

  // the wave's 16 query rows as B fragments of v_mfma_f32_16x16x32_bf16:
  // lane -> row r16, dims 32ks + 8q4 + i
  u32x4_t qf[KS];
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
    // row 0 of request qb stands in for padding rows: always a valid address
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)qb * a.Hq + head) * DK + 8 * q4;
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
  // lane i fetching item 64k + i.
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
  // every wave converts NIT blocks (waves with fewer repeat their last one:
  // same bytes to the same place), so the code is branch-free and can be
  // interleaved with the products of the current tile
  constexpr int NIT = (NBLK + kWaves - 1) / kWaves;
  auto convert_tile = [&](uint16_t* dstbuf) {
    // recomputed per tile rather than kept live across it
    int lane_r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_r) : "v"(lane));
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      int k = wave + kWaves * it;
      k = (k < NBLK) ? k : k - kWaves;
      if constexpr (KT == LK_FP8) {
        // 8 codes (one bf16 chunk) per lane and pass: consecutive lanes
        // write consecutive chunks of a row
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int j = 128 * k + 64 * hh + lane_r;  // 8-code group of the tile
          const int tt = j / (DK / 8), q = j - tt * (DK / 8);
          const u32x2_t x = reinterpret_cast<const u32x2_t*>(sraw)[j];
          uint32_t w[4];
          fp8x4_dequant_bf16(x[0], a.k_scale, w[0], w[1]);
          fp8x4_dequant_bf16(x[1], a.k_scale, w[2], w[3]);
          *reinterpret_cast<u32x4_t*>(dstbuf + tt * DK + 8 * swz(tt, q)) = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      } else {
        const int c = 64 * k + lane_r;
        const int tt = c / RCH, rc = c - tt * RCH;
        *reinterpret_cast<u32x4_t*>(dstbuf + tt * DK + 8 * swz(tt, rc)) = sraw[c];
      }
    }
  };
  f32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float run_m = -INFINITY, run_l = 0.f;

  // Per-lane LDS element offsets within the tile. The swizzle permutes the
  // low three bits of the chunk index, so each read is a per-lane base plus
  // a compile-time offset:
  //   K fragment (tb, ks): token 16tb + r16, chunk 4ks + q4
  //     -> (16tb + r16)*DK + 64(ks/2) + 8(q4 ^ f(r16) ^ 4(ks%2));
  //   V^T fragment of dims 16db..16db+15: tokens 4q4 + e and 16 + 4q4 + e,
  //     lane r16 of the group addressing token 4q4 + r16/4 at dims
  //     16db + 4(r16%4), chunk 2db + (r16%4)/2
  //     -> tok*DK + 64(db/4) + 8((2(db%4)) ^ z) + 4(r16%2), z = (r16%4)/2 ^ f(tok).
  // The chunk term occupies bits 3..5 of an offset (DK is a multiple of 64),
  // so the variants for ks odd and db % 4 = c are XORs of one register with
  // 32 and 16c, redone per tile instead of held.
  const int fk = (5 * (r16 >> 1)) & 7;
  const int kofs = r16 * DK + 8 * (q4 ^ fk);
  const int v_tok = 4 * q4 + (r16 >> 2);
  const int v_z = ((r16 & 3) >> 1) ^ ((5 * (v_tok >> 1)) & 7);
  const int vofs = v_tok * DK + 8 * v_z + 4 * (r16 & 1);
  static_assert(DK % 64 == 0, "chunk bits below the token stride");

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query fragments have landed
  __syncthreads();                     // page ids visible
  const int n_tt = (end > start) ? (end - start + kTT - 1) / kTT : 0;
  if (n_tt > 0) {
    fetch_tile(start);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    convert_tile(sk0);
    if (n_tt > 1) fetch_tile(start + kTT);
  }
  __syncthreads();

  // S^T = K . Q^T for one tile: block tb, lane -> query row r16, tokens
  // 16tb + 4q4 + j
  auto s_phase = [&](const uint16_t* tile_k, f32x4_t (&s)[2]) {
    constexpr int KP = 2, NK = 2 * KS;
    u32x4_t kf[NK];
    int k0;
    asm volatile("v_mov_b32 %0, %1" : "=v"(k0) : "v"(kofs));
    const int k1 = k0 ^ 32;
    auto kread = [&](int i) {
      const int tb = i / KS, ks = i - tb * KS;
      return *reinterpret_cast<const u32x4_t*>(tile_k + 16 * tb * DK + ((ks & 1) ? k1 : k0) +
                                               64 * (ks >> 1));
    };
    s[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KP; ++i) kf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (i + KP < NK) kf[i + KP] = kread(i + KP);
      const int tb = i / KS, ks = i - tb * KS;
      s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[i]), as_bf16x8(qf[ks]), s[tb],
                                                      0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, KP, 0);
#pragma unroll
    for (int i = 0; i < NK - KP; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, KP, 0);
  };

  // online softmax of one tile's scores: rescales the running state and
  // returns P^T as the B operand of the PV product (k slots 8q4 + i are
  // tokens 4q4 + i (i < 4) and 16 + 4q4 + i - 4), split into bf16 hi + lo
  // parts (lo = P - hi, rounded) so that the product keeps P to about 16
  // bits (one bf16 rounding of P alone errs by up to 2^-9 per weight)
  auto softmax = [&](f32x4_t (&s)[2], int t0, bf16x8_t& plo) {
    // row max over the four lane groups, in scaled log2 units; a full tile
    // scales inside the exponent below, the last tile masks first
    float cs = a.scale_log2, mx;
    if (t0 + kTT <= end_lo) {
      float hi = fmaxf(s[0][0], s[1][0]), lo = fminf(s[0][0], s[1][0]);
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        hi = fmaxf(hi, fmaxf(s[0][j], s[1][j]));
        lo = fminf(lo, fminf(s[0][j], s[1][j]));
      }
      mx = (cs >= 0.f ? hi : lo) * cs;
    } else {
      mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = t0 + 16 * tb + 4 * q4 + j;
          s[tb][j] = (t < my_end) ? s[tb][j] * cs : -INFINITY;
          mx = fmaxf(mx, s[tb][j]);
        }
      cs = 1.f;
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
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
    uint32_t pw[4], pl[4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[tb][j], cs, -mu));
        const float p1 = fast_exp2(__builtin_fmaf(s[tb][j + 1], cs, -mu));
        run_l += p0 + p1;
        const uint32_t hw = pack_bf16x2_rne(p0, p1);
        pw[2 * tb + (j >> 1)] = hw;
        pl[2 * tb + (j >> 1)] = pack_bf16x2_rne(p0 - bf16_lo(hw), p1 - bf16_hi(hw));
      }
    plo = as_bf16x8(u32x4_t{pl[0], pl[1], pl[2], pl[3]});
    return as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
  };

  // O^T += V^T . P^T, V^T fragments by transposing loads issued VP products
  // ahead
  auto pv_phase = [&](const uint16_t* tile_k, bf16x8_t pb, bf16x8_t plo) {
    constexpr int VP = 2;
    u32x4_t vf[DB];
    int v0;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v0) : "v"(vofs));
    auto vread = [&](int db) {
      const uint16_t* p0 = tile_k + (v0 ^ (16 * (db & 3))) + 64 * (db >> 2);
      const u32x2_t v0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0));
      const u32x2_t v1 =
          __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p0 + 16 * DK)));
      return u32x4_t{v0[0], v0[1], v1[0], v1[1]};
    };
#pragma unroll
    for (int i = 0; i < VP; ++i) vf[i] = vread(i);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + VP < DB) vf[db + VP] = vread(db + VP);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[db]), pb, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[db]), plo, acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * VP, 0);
#pragma unroll
    for (int i = 0; i < DB - VP; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2 * VP, 0);
  };

  // Interval i (one barrier each): tile i is read from buffer i % 3; tile
  // i + 1 is converted into buffer (i + 1) % 3 by the waves that fetched its
  // blocks, each of which then fetches its blocks of tile i + 2 into the raw
  // buffer once its own LDS reads of the interval are issued (the compiler
  // makes LDS stores and transposing LDS loads wait for global->LDS loads in
  // flight). The second half of the waves runs each tile's PV product one
  // interval late, converting first: on each SIMD one wave's softmax and
  // conversion then fall beside the other's products. Buffer (i - 1) % 3
  // stays intact until interval i + 1 converts into it.
  const bool lagged = kStagger && wave >= kWaves / 2;  // wave-uniform
  bf16x8_t pb{}, plo{};  // P^T of the last tile (lagged waves: not yet applied)
  auto interval = [&](int i, const uint16_t* cur, uint16_t* next, const uint16_t* prev) {
    const int t0 = start + i * kTT;
    auto convert_next = [&]() {
      if (i + 1 < n_tt) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile i + 1 has landed
        convert_tile(next);
      }
    };
    if (lagged) {
      convert_next();
      if (i > 0) pv_phase(prev, pb, plo);
    }
    f32x4_t s[2];
    s_phase(cur, s);
    if (lagged && i + 2 < n_tt) fetch_tile(t0 + 2 * kTT);
    pb = softmax(s, t0, plo);
    if (!lagged) {
      convert_next();
      pv_phase(cur, pb, plo);
      if (i + 2 < n_tt) fetch_tile(t0 + 2 * kTT);
    }
    lds_barrier();  // tile i read by all waves; tile i + 1 staged
  };
  for (int i = 0; i < n_tt; i += 3) {
    interval(i, sk0, sk1, sk2);
    if (i + 1 < n_tt) interval(i + 1, sk1, sk2, sk0);
    if (i + 2 < n_tt) interval(i + 2, sk2, sk0, sk1);
  }
  if (lagged && n_tt > 0) {  // no fetch in flight here
    const int last = (n_tt - 1) % 3;
    pv_phase(last == 0 ? sk0 : last == 1 ? sk1 : sk2, pb, plo);
  }

  // row sum over the lane groups, normalized partial and its LSE
  float l = run_l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (my_row < nrows) {
    const int m = my_row / a.G, g = my_row % a.G;
    const size_t o = state_index(a, stacked, mbase, b, p, m, h * a.G + g);
    float* dst = a.v_out + o * DV + 4 * q4;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<float4*>(dst + 16 * db) =
          make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
    if (q4 == 0) a.lse_out[o] = (l > 0.f) ? run_m + log2f(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp8 latent pools: 4 waves (one per SIMD), 32 query rows per wave.
//
// Every K or V^T fragment read from LDS feeds a 32-row product
// (v_mfma_f32_32x32x16_bf16): half the LDS bytes per flop of 16-row
// fragments. With 128 rows and 576-wide rows the products are bound by LDS
// read bandwidth (128 B per clock per CU) rather than by the matrix cores.
// Each wave keeps Q^T for its 32 rows (36 B fragments, 144 registers) and
// O^T = 512 dims x 32 rows (16 blocks of 32 x 32, the 256 accumulator
// registers) for the whole partition: one wave per SIMD has the 512
// registers for both.
//   * S^T = K . Q^T per 32-token tile: A = K (32 tokens x 16 dims, one
//     16-byte LDS read per lane), B = Q^T (16 dims x 32 rows); lane j holds
//     S^T[token 8(r/4) + 4(j/32) + r%4][row j%32] in register r.
//   * O^T += V^T . P^T in two 16-token k-steps: B = P^T straight from the S^T
//     registers (k slot i of lane j = register 8kk + i, i.e. tokens
//     16kk + 4(j/32) + {0..3}, then 16kk + 8 + 4(j/32) + {0..3}); A = V^T
//     (32 dims x those 16 tokens) from the row-major tile by two transposing
//     loads (ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives
//     element i%4 of the 8 bytes addressed by lane 4e + i/4 as its element
//     e; lane 16g + 4e + s addresses token 4(g/2) + e, dims 16(g%2) + 4s).
//   * Tiles are stored bf16 [token][576] with 16-byte chunk c of token t at
//     position c ^ f(t) within its aligned group of 8 chunks, f(t) bits:
//     b0 = t2, b1 = t0 ^ t3, b2 = t1. Rows are 1152 bytes apart, so with
//     LDS banks 128 or 256 bytes wide alike, the K reads (8 or 16
//     consecutive tokens, one chunk), the transposing reads (4 tokens x 2
//     or x 4 chunks per bank cycle) and the dequantized stores are free of
//     bank conflicts (f was chosen by checking every access pattern under
//     both bank widths).
// Fetch: the fp8 rows of tile i + 2 go through registers during interval
// i, lane L taking token L/8 and 8-code units (L%8) + 8k, k < 9 (each fetch
// instruction reads 64 contiguous bytes per token, each LDS store fills one
// 128-byte bank line per token); each lane dequantizes its own units
// (RNE_bf16(f32(x) * scale)) into a bf16 LDS buffer one interval later. No
// global->LDS loads, so no LDS access waits for a fetch.
// Interval i (one barrier; three buffers): the S^T chain of tile i (36
// dependent products; gfx950 issues such a chain at the full rate)
// interleaved with O^T of tile i - 1 (32 products on 16 independent
// accumulators, k-step major), which spreads the K and V^T reads evenly;
// the dequantization of tile i + 1 (two vector operations after each
// product) and the fetch of tile i + 2
// spread over the same loop; then the softmax of tile i. The S^T products
// are written as inline asm with VGPR operands and the O^T products with
// accumulation-register operands: the compiler otherwise gives every
// product's accumulator the same register file and has no room for both.
// The query fragments are fetched first, so that their issue (36 loads of
// 32 rows each) overlaps the page-table reads.
// Measured (32 requests x 16384 fp8 tokens, 2048-token partitions): 160-166
// us per launch against 195 us for the 8-wave kernel above; with the
// matrix cores 40% busy by counter, LDS 26% busy, no bank conflicts. Cycle
// stamps (s_memtime) per workgroup: prologue about 7 us, tile loop about
// 130 us, the partial's stores 12 us; the clock under this load is 1.8-2.0
// GHz, not 2.4. An interval takes about 4,000 cycles against 2,176 of
// products: the launch is bound by the one wave's instruction issue (about
// 430 other instructions per interval: the dequantization, the softmax,
// LDS reads and waits), and with one wave per SIMD no other wave fills
// the issue slots they take.
// Softmax reference: a row's scores are exponentiated against a fixed
// reference, its maximum over the first tile it sees, and the accumulators
// are never rescaled (a VALU rescale of accumulator registers costs the
// registers the products need). A later score more than kRefL (log2 units)
// above the reference would overflow that scheme: then the whole workgroup
// restarts the partition with the raised reference, accumulators zeroed. The
// result is the same exact softmax either way; the restart costs a second
// pass and happens only for scores that grow by more than 2^kRefL within a
// partition.
// ---------------------------------------------------------------------------

typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr float kRefL = 16.f;

// chunk swizzle of token t (see above)
__device__ __forceinline__ int fswz(int t) {
  return ((t >> 2) & 1) | (((t ^ (t >> 3)) & 1) << 1) | (((t >> 1) & 1) << 2);
}

template <int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void partial_latent_fp8_kernel(const PartialArgs a) {
  constexpr int NW = 4;                   // waves, one per SIMD
  constexpr int RW = 32;                  // query rows per wave
  constexpr int ROWS = NW * RW;           // 128
  constexpr int NT = 64 * NW;
  constexpr int KS = DK / 16;             // k-steps of S^T (16 dims)
  constexpr int DB = DV / 32;             // 32-dim output blocks
  constexpr int RB = DK * 2;              // bytes of a bf16 tile row
  constexpr int CPR = DK / 8;             // 16-byte bf16 chunks (8-code units) per row
  constexpr int UPL = CPR / 8;            // units per lane and tile
  static_assert(CPR % 8 == 0 && NT == 8 * kTT, "8 lanes per token, whole units per lane");
  static_assert(RB % 128 == 0 && DK % 64 == 0 && DV % 64 == 0 && DV <= DK, "latent shapes");

  // three bf16 tile buffers, chosen at run time (no global->LDS loads, so
  // nothing needs the compiler to tell them apart)
  __shared__ __align__(16) uint16_t sbuf[3][kTT * DK];
  __shared__ int sm_pid[kMaxPagesL];
  __shared__ int sm_restart;

  const int n_tiles = (a.max_rows + ROWS - 1) / ROWS;
  int unit, tile;
  xcd_unit_tile(blockIdx.x, n_tiles, unit, tile);
  {
    // Workgroups are dealt to the 8 XCDs round robin by block index. With
    // one tile per unit and a unit count divisible by 8, XCD x takes the
    // consecutive units [x units/8, (x+1) units/8): a request's partitions
    // (consecutive units reading the same query rows) then share one L2.
    const int units = a.num_parts * a.Hkv;
    if (n_tiles == 1 && (units & 7) == 0) unit = (blockIdx.x & 7) * (units >> 3) + (blockIdx.x >> 3);
  }
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
  const int row0 = tile * ROWS;
  if (row0 >= nrows) return;  // uniform

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hf = lane >> 5;    // lane half
  const int n32 = lane & 31;   // query row of the wave (MFMA column) / token of a K read
  const int my_row = row0 + RW * wave + n32;
  const bool live_wave = row0 + RW * wave < nrows;  // uniform over the wave

  // Q^T fragments: lane -> row n32, dims 16ks + 8hf + 0..7. Issued before
  // the page-table reads below, which their issue then overlaps.
  u32x4_t qf[KS];
  if (!stacked && a.Hkv == 1) {
    // One latent KV head: the view's rows are consecutive rows of q (row r
    // of request b is q row b T Hq + r). Each wave reads its 32 rows in
    // thirds of the dims with loads whose lanes cover consecutive 16-byte
    // chunks of a row (a few cache lines per load instead of 32), stages
    // them in its own part of tile buffers 1-2 (free until the tile loop;
    // rows padded to 400 bytes, so the fragment reads of 32 rows hit
    // distinct banks) and reads its fragments back. Rows past the view
    // repeat its last row and are zeroed.
    constexpr int QSTR = 400, NQL = RW * 24 / 64;  // row stride; 16-byte loads per lane and third
    static_assert(DK == 576 && (RW * 24) % 64 == 0, "thirds of 192 dims, whole loads");
    static_assert(NW * RW * QSTR <= 2 * (int)sizeof(sbuf[0]), "staging fits buffers 1-2");
    const char* q0 = reinterpret_cast<const char*>(a.q) +
                     ((size_t)b * a.q_tokens * a.Hq) * RB;
    char* stage = reinterpret_cast<char*>(sbuf) + sizeof(sbuf[0]) + wave * (RW * QSTR);
    const bool live = my_row < nrows;
#pragma unroll
    for (int p3 = 0; p3 < 3; ++p3) {
      u32x4_t raw[NQL];
#pragma unroll
      for (int i = 0; i < NQL; ++i) {
        const int c = 64 * i + lane, rr = c / 24, cq = c % 24;
        const int row = min(row0 + RW * wave + rr, nrows - 1);
        raw[i] = *reinterpret_cast<const u32x4_t*>(q0 + (size_t)row * RB + 384 * p3 + 16 * cq);
      }
#pragma unroll
      for (int i = 0; i < NQL; ++i) {
        const int c = 64 * i + lane, rr = c / 24, cq = c % 24;
        *reinterpret_cast<u32x4_t*>(stage + rr * QSTR + 16 * cq) = raw[i];
      }
      // a wave's LDS operations complete in order: these reads see the
      // stores above, and the next third's stores follow them
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(stage + n32 * QSTR + 16 * (2 * k + hf));
        qf[12 * p3 + k] = live ? x : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  } else {
    int qb = b, head = 0;
    const bool live = my_row < nrows;
    if (live) {
      const int m = my_row / a.G, g = my_row % a.G;
      qb = query_row(a, stacked, mbase, b, m);
      head = h * a.G + g;
    }
    // row 0 of request qb stands in for padding rows: always a valid address
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)qb * a.Hq + head) * DK + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
      qf[ks] = live ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  int page0, start, end;
  part_range(a, b, p, page0, start, end);
  // causal rows: the tile loop stops at the last owned row's end; every
  // owned row sees at least the positions below end_lo (uniform)
  const int end_lo = min(end, visible_end(a, b, row0 / a.G));
  end = min(end, visible_end(a, b, (min(row0 + ROWS, nrows) - 1) / a.G));
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
  if (tid == 0) sm_restart = 0;
  const int my_end = min(end, visible_end(a, b, min(my_row, nrows - 1) / a.G));

  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride;
  const long long kb_stride = a.k_bstride;

  // Unit k of lane tid: token tt = tid / 8, 8 codes at dims 8c, c = tid % 8
  // + 8k, stored at chunk position 8k + ((tid % 8) ^ f(tt)); a tile never
  // crosses a page (P is a multiple of the tile); rows past the end repeat
  // the last token.
  const int u_tt = tid >> 3;
  const int u_lds = u_tt * RB + 16 * ((tid & 7) ^ fswz(u_tt));  // + 128 k
  auto fetch = [&](int t0, u32x2_t (&F)[UPL]) {
    const int pid = __builtin_amdgcn_readfirstlane(sm_pid[(t0 >> shift) - pg_first]);
    const char* pbase = kbase + pid * kb_stride + (long long)(t0 & pmask) * DK;
    const char* src = pbase + min(u_tt, end - 1 - t0) * DK + 8 * (tid & 7);  // + 64 k
#pragma unroll
    for (int k = 0; k < UPL; ++k) F[k] = *reinterpret_cast<const u32x2_t*>(src + 64 * k);
  };
  auto convert = [&](const u32x2_t (&F)[UPL], uint16_t* dst) {
    char* d = reinterpret_cast<char*>(dst) + u_lds;
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      uint32_t w[4];
      fp8x4_dequant_bf16(F[k][0], a.k_scale, w[0], w[1]);
      fp8x4_dequant_bf16(F[k][1], a.k_scale, w[2], w[3]);
      *reinterpret_cast<u32x4_t*>(d + 128 * k) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  };

  // Per-lane LDS byte offsets (chunk bits XOR-swizzled by token):
  //   K read of k-step ks: token n32, chunk 2ks + hf -> position
  //     8(ks/4) + (2(ks%4) ^ z), z = hf ^ f(n32):
  //     kofs ^ 32(ks%4) + 128(ks/4), kofs = n32*RB + 16z;
  //   V^T reads of block db, k-step kk: token 16kk + T0 (+ 8), chunk
  //     4db + c, c = 2(g%2) + s/2 -> position 8(db/2) + (4(db%2) ^ x),
  //     x = c ^ f(T0) (f(T0 + 8) = f(T0) ^ 2, f(T + 16) = f(T)):
  //     vofs ^ 64(db%2) (^ 32) + 128(db/2) + (16kk (+8)) RB,
  //     vofs = T0*RB + 16x + 8(s%2), T0 = 4(g/2) + e.
  const int kofs = n32 * RB + 16 * (hf ^ fswz(n32));
  int vofs;
  {
    const int g = lane >> 4, e = (lane >> 2) & 3, s = lane & 3;
    const int T0 = 4 * (g >> 1) + e;
    const int x = (2 * (g & 1) + (s >> 1)) ^ fswz(T0);
    vofs = T0 * RB + 16 * x + 8 * (s & 1);
  }

  f32x16_t acc[DB];
  float ref = -INFINITY, run_l = 0.f;  // per row (both lane halves agree)

  // One step of the S^T chain, written out so that the accumulator stays in
  // ordinary VGPRs while the O^T accumulators fill the 256 accumulation
  // registers (the compiler otherwise puts every product's accumulator in
  // the accumulation file and has no room for both). gfx950 interlocks a
  // product on its predecessor's result (the chain needs no wait states),
  // the first step starts from the inline constant 0 (no VALU write of the
  // accumulator is ever read), and after the last step the 12 wait states
  // an XDL result needs before a VALU reads it are inserted here, since the
  // compiler does not see this product.
  auto qk_step = [&](int st, const u32x4_t& kfr, const u32x4_t& qfr, f32x16_t& s) {
    if (st == 0) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(kfr), "v"(qfr));
    } else if (st < KS - 1) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kfr), "v"(qfr));
    } else {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 4"
                   : "+v"(s) : "v"(kfr), "v"(qfr));
    }
  };

  // One O^T product, written out so that its accumulator stays in the
  // accumulation registers. The accumulators are written only by these
  // products (zeroed once per pass, followed by the wait states a product
  // reading them needs) and read only after the tile loop (after the wait
  // states an XDL result needs). P^T comes from VALU instructions: the first
  // product of an interval waits the 2 states an XDL source written by VALU
  // needs.
  auto pv_step = [&](int st, const u32x4_t& vfr, const bf16x8_t& pbr, f32x16_t& o) {
    if (st == 0) {
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(o) : "v"(vfr), "v"(pbr));
    } else {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(vfr), "v"(pbr));
    }
  };

  // V^T fragment i = DB kk + db (32 dims x 16 tokens) of the tile at tv,
  // from the lane's offset v0 (see above)
  auto vread_from = [&](const char* tv, int v0, int i) {
    const int kk = i / DB, db = i % DB;
    const char* p0 = tv + (v0 ^ (64 * (db & 1))) + 128 * (db >> 1) + 16 * kk * RB;
    const char* p1 = tv + (v0 ^ (64 * (db & 1) + 32)) + 128 * (db >> 1) + (16 * kk + 8) * RB;
    const u32x2_t x0 = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0));
    const u32x2_t x1 = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1));
    return u32x4_t{x0[0], x0[1], x1[0], x1[1]};
  };

  // The O^T products of the last tile alone, after the tile loop: no S^T
  // product or dequantization is left to pair them with.
  auto pv_tail = [&](const uint16_t* prev, const bf16x8_t (&pb)[2]) {
    constexpr int VP = 2, NPV = 2 * DB;
    const char* tv = reinterpret_cast<const char*>(prev);
    int v0;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v0) : "v"(vofs));
    u32x4_t vf[VP + 1];
#pragma unroll
    for (int q = 0; q < VP; ++q) vf[q] = vread_from(tv, v0, q);
#pragma unroll
    for (int st = 0; st < NPV; ++st) {
      if (st + VP < NPV) vf[(st + VP) % (VP + 1)] = vread_from(tv, v0, st + VP);
      pv_step(st, vf[st % (VP + 1)], pb[st / DB], acc[st % DB]);
    }
  };

  // One interval's products: S^T of tile `cur` (a chain of KS dependent
  // MFMAs) interleaved with O^T += V^T . P^T of the tile before it (2 DB
  // MFMAs on DB independent accumulators, k-step major), which spreads the
  // K and V^T reads evenly; the dequantization of the next tile and the
  // fetch of the one after it are spread over the same loop, one unit every
  // few steps. K fragments are read KP steps ahead, V^T fragments VP
  // steps ahead, into rings of registers (deeper rings measured no faster).
  // The dequantization and fetch always run (past the last tile they repeat
  // it: same bytes, unused buffer).
  auto products = [&](const uint16_t* cur, const uint16_t* prev, const bf16x8_t (&pb)[2],
                      f32x16_t& s, uint16_t* next, u32x2_t (&F)[UPL], int t_fetch) {
    constexpr int KP = 2, VP = 2, NPV = 2 * DB;
    constexpr int STEPS = KS > NPV ? KS : NPV;
    constexpr int CONV_EVERY = STEPS / UPL;
    static_assert(CONV_EVERY >= 1, "unit spacing");
    const char* tk = reinterpret_cast<const char*>(cur);
    const char* tv = reinterpret_cast<const char*>(prev);
    int k0, v0;
    asm volatile("v_mov_b32 %0, %1" : "=v"(k0) : "v"(kofs));
    asm volatile("v_mov_b32 %0, %1" : "=v"(v0) : "v"(vofs));
    auto kread = [&](int ks) {
      return *reinterpret_cast<const u32x4_t*>(tk + (k0 ^ (32 * (ks & 3))) + 128 * (ks >> 2));
    };
    auto vread = [&](int i) { return vread_from(tv, v0, i); };  // i = DB kk + db
    // the tile after next (page uniform over the tile)
    const int pid = __builtin_amdgcn_readfirstlane(sm_pid[(t_fetch >> shift) - pg_first]);
    const char* src = kbase + pid * kb_stride + (long long)(t_fetch & pmask) * DK +
                      min(u_tt, end - 1 - t_fetch) * DK + 8 * (tid & 7);
    char* dst = reinterpret_cast<char*>(next) + u_lds;
    u32x4_t kf[KP + 1], vf[VP + 1];
#pragma unroll
    for (int i = 0; i < KP; ++i) kf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < VP; ++i) vf[i] = vread(i);
    // Dequantization of unit k: 16 vector operations (the unit's two 4-code
    // words in turn: both halves widened to binary32, exactly; four products
    // with the scale; two RNE roundings to bf16 pairs: RNE_bf16(RNE_f32(x *
    // scale)), the instructions fp8x4_dequant_bf16 compiles to), spread
    // evenly over the products of the unit's steps. Each is its own asm
    // statement so that it stays where it is put: as ordinary code the
    // compiler gathers a unit's operations between two products, and the
    // matrix core then waits for them.
    f32x2_t dq_lo, dq_hi;
    float dq_m[4];
    uint32_t dq_w[4];
    const float scl = a.k_scale;
    auto dq_op = [&](int k, int j) {
      const uint32_t x = F[k][j >> 3];
      switch (j & 7) {
        case 0: asm volatile("v_cvt_pk_f32_fp8_e32 %0, %1" : "=v"(dq_lo) : "v"(x)); break;
        case 1: asm volatile("v_cvt_pk_f32_fp8_sdwa %0, %1 src0_sel:WORD_1" : "=v"(dq_hi) : "v"(x)); break;
        case 2: asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(dq_m[0]) : "s"(scl), "v"(dq_lo[0])); break;
        case 3: asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(dq_m[1]) : "s"(scl), "v"(dq_lo[1])); break;
        case 4: asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(dq_m[2]) : "s"(scl), "v"(dq_hi[0])); break;
        case 5: asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(dq_m[3]) : "s"(scl), "v"(dq_hi[1])); break;
        case 6:
          asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(dq_w[2 * (j >> 3)]) : "v"(dq_m[0]), "v"(dq_m[1]));
          break;
        default:
          asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2"
                       : "=v"(dq_w[2 * (j >> 3) + 1]) : "v"(dq_m[2]), "v"(dq_m[3]));
      }
    };
    // products in steps [t0, t1), and unit k's share of its operations for
    // the idx-th product of its steps
    auto n_products = [](int t0, int t1) {
      int n = 0;
      for (int t = t0; t < t1; ++t) n += (t < KS) + (t < NPV);
      return n;
    };
    auto dq_share = [&](int st, int slot) {
      const int k = st / CONV_EVERY;
      if (k >= UPL) return;
      const int t0 = k * CONV_EVERY;
      const int n = n_products(t0, t0 + CONV_EVERY);
      const int idx = n_products(t0, st) + slot;
      for (int j = 16 * idx / n; j < 16 * (idx + 1) / n; ++j) dq_op(k, j);
    };
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      if (st < KS) {
        if (st + KP < KS) kf[(st + KP) % (KP + 1)] = kread(st + KP);
        qk_step(st, kf[st % (KP + 1)], qf[st], s);
        // the previous unit's LDS store and the next fetch into its
        // registers come one product after that unit's last operation (in
        // the step before), so that the store does not wait on its result
        if (st % CONV_EVERY == 0 && st > 0 && st / CONV_EVERY - 1 < UPL) {
          const int k = st / CONV_EVERY - 1;
          *reinterpret_cast<u32x4_t*>(dst + 128 * k) = u32x4_t{dq_w[0], dq_w[1], dq_w[2], dq_w[3]};
          F[k] = *reinterpret_cast<const u32x2_t*>(src + 64 * k);
        }
        dq_share(st, 0);
      }
      if (st < NPV) {
        if (st + VP < NPV) vf[(st + VP) % (VP + 1)] = vread(st + VP);
        pv_step(st, vf[st % (VP + 1)], pb[st / DB], acc[st % DB]);
        dq_share(st, st < KS ? 1 : 0);
      }
    }
    {
      static_assert(STEPS / CONV_EVERY == UPL, "the last unit ends with the loop");
      constexpr int k = UPL - 1;
      *reinterpret_cast<u32x4_t*>(dst + 128 * k) = u32x4_t{dq_w[0], dq_w[1], dq_w[2], dq_w[3]};
      F[k] = *reinterpret_cast<const u32x2_t*>(src + 64 * k);
    }
  };

  // online softmax of one tile's scores against the row's reference; a
  // score far above it asks for a restart with the reference raised.
  // Returns P^T for the two k-steps of the PV product.
  auto softmax = [&](f32x16_t& s, int t0, int pass, bf16x8_t (&pb)[2]) {
    float cs = a.scale_log2, mx;
    if (t0 + kTT <= end_lo) {
      float hi = s[0], lo = s[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) {
        hi = fmaxf(hi, s[j]);
        lo = fminf(lo, s[j]);
      }
      mx = (cs >= 0.f ? hi : lo) * cs;
    } else {
      mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + 8 * (j >> 2) + 4 * hf + (j & 3);
        s[j] = (t < my_end) ? s[j] * cs : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      cs = 1.f;
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(f32_bits(mx), f32_bits(mx), false, false);
      mx = fmaxf(bits_f32(sw[0]), bits_f32(sw[1]));  // over lanes l and l ^ 32
    }
    if (ref == -INFINITY) ref = mx;  // the first visible tile sets the reference
    if (__builtin_expect(__any(mx > ref + kRefL), 0)) {
      ref = fmaxf(ref, mx);
      sm_restart = pass + 1;
    }
    const float mu = (ref == -INFINITY) ? 0.f : ref;
    uint32_t pw[8];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[j], cs, -mu));
      const float p1 = fast_exp2(__builtin_fmaf(s[j + 1], cs, -mu));
      run_l += p0 + p1;
      pw[j >> 1] = pack_bf16x2_rne(p0, p1);
    }
    pb[0] = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
    pb[1] = as_bf16x8(u32x4_t{pw[4], pw[5], pw[6], pw[7]});
  };

  const int n_tt = (end > start) ? (end - start + kTT - 1) / kTT : 0;
  const int t_last = start + max(n_tt - 1, 0) * kTT;  // first token of the last tile
  __syncthreads();  // page ids and the restart flag visible
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = f32x16_t{};
      asm volatile("" : "+a"(acc[db]));  // zeroed in the accumulation registers
    }
    asm volatile("s_nop 4" ::: "memory");  // VALU writes before a product reads them
    run_l = 0.f;
    u32x2_t F[UPL];
    if (n_tt > 0) {
      fetch(start, F);
      convert(F, sbuf[0]);
      fetch(min(start + kTT, t_last), F);
    }
    lds_barrier();
    bool restart = false;
    bf16x8_t pb[2] = {};
    // interval i: tile i + 1 dequantized into buffer (i + 1) % 3 (and tile
    // i + 2 fetched), S^T of tile i from buffer i % 3 with O^T of tile
    // i - 1 from buffer (i + 2) % 3, then the softmax of tile i; the O^T
    // products of the last tile follow the loop alone.
    // Every interval runs the same products (one code path keeps the
    // registers the allocator needs to the products'): before the first
    // tile the O^T product reads tile 0 with P = 0 (it adds exact zeros);
    // the last interval dequantizes a repeat of the last tile into an
    // unused buffer. Waves whose rows are all padding compute with zero
    // queries and write nothing.
    for (int i = 0, bi = 0; i < n_tt && !restart; ++i, bi = (bi == 2) ? 0 : bi + 1) {
      const int bp = bi == 0 ? 2 : bi - 1;
      const uint16_t* cur = sbuf[bi];
      const uint16_t* prev = sbuf[i > 0 ? bp : bi];
      uint16_t* next = sbuf[bi == 2 ? 0 : bi + 1];
      const int t_fetch = min(start + (i + 2) * kTT, t_last);
      f32x16_t s;
      products(cur, prev, pb, s, next, F, t_fetch);
      if (live_wave) softmax(s, start + i * kTT, pass, pb);
      lds_barrier();  // tiles i - 1 and i read by all waves; tile i + 1 staged
      restart = sm_restart > pass;  // uniform over the workgroup
    }
    if (!restart && n_tt > 0) pv_tail(sbuf[(n_tt - 1) % 3], pb);
    if (!restart) break;
  }
  // the last products' results before any VALU reads them
  asm volatile("s_nop 7\n\ts_nop 4" ::: "memory");

  // row sum over the two lane halves, normalized partial and its LSE
  float l = run_l;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(f32_bits(l), f32_bits(l), false, false);
    l = bits_f32(sw[0]) + bits_f32(sw[1]);
  }
  if (my_row < nrows) {
    const int m = my_row / a.G, g = my_row % a.G;
    const size_t o = state_index(a, stacked, mbase, b, p, m, h * a.G + g);
    float* dst = a.v_out + o * DV + 4 * hf;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 32 * db + 8 * q) =
            make_float4(acc[db][4 * q] * inv, acc[db][4 * q + 1] * inv, acc[db][4 * q + 2] * inv,
                        acc[db][4 * q + 3] * inv);
    if (hf == 0) a.lse_out[o] = (l > 0.f) ? ref + log2f(l) : -INFINITY;
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
  const bool fp8 = a.kv_dtype == PDK_FP8_E4M3;
  if (!fp8 && a.kv_dtype != PDK_BF16) return PDK_OK;
  if (a.S / a.P + 1 > kMaxPagesL)
    return fail(PDK_ERR_UNSUPPORTED, "partition of %d tokens spans more than %d pages", a.S,
                kMaxPagesL - 1);
  *handled = true;
  const long long units = (long long)a.num_parts * a.Hkv;
  // Rows per workgroup: 128 (the fp8 kernel always; the bf16 kernel's 8
  // waves). A bf16 launch whose 128-row grid would leave CUs idle (a short
  // suffix range: few partitions) takes 64-row workgroups of 4 waves
  // instead, twice the workgroups for the same rows, and so does one of at
  // most 64 rows (no dead waves).
  int rows = 128, threads = 256;
  LatentFn fn = partial_latent_fp8_kernel<576, 512>;
  if (!fp8) {
    const long long blocks128 = xcd_grid_blocks(units, (a.max_rows + 127) / 128);
    const bool narrow = a.max_rows <= 64 || blocks128 < kChipCUs;
    rows = narrow ? 64 : 128;
    threads = narrow ? 256 : 512;
    fn = narrow ? partial_latent_kernel<576, 512, LK_BF16, 4>
                : partial_latent_kernel<576, 512, LK_BF16, 8>;
  }
  const int n_tiles = (a.max_rows + rows - 1) / rows;
  const long long blocks = xcd_grid_blocks(units, n_tiles);
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "latent partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
