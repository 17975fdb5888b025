// Paged split-KV partial attention for bf16 K/V pools of head dim 128 on
// the matrix cores, with K/V tiles streamed into LDS by gfx950's
// global->LDS loads [cascade-PR = mlxcel pull request "perf(core): compute
// shared prompt prefixes once per decode batch", "The decomposition":
// each (request, page tile) yields a partial (V, LSE); level 0 is the same
// launch with the members' query rows stacked per KV head]. Same contract
// as the other partial kernels: one normalized partial and its log2 LSE per
// (request, partition, query row).
//
// Workgroup = NW waves, 16 query rows each, all of one KV head; they share
// the K/V tiles of their (request, partition). A tile of TT tokens is K
// [TT][128] plus V [TT][128] in bf16; NS tile stages form a ring that the
// global->LDS loads (16 bytes per lane, lane i at base + 16i) fill NS-1
// tiles ahead of the products, so no registers hold rows in flight and the
// loads are never converted. Per tile:
//   * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16: A = 16 K rows from LDS,
//     B = the wave's 16 query rows (registers, loaded once);
//   * online softmax per query row in log2 units (lazy reference maximum,
//     raised only past +8), row max across the four lane groups;
//   * O^T += V^T . P^T: A = 16 value dims x 32 tokens read from the
//     row-major V tile with the transposing LDS load (ds_read_b64_tr_b16), B
//     = P^T straight from the S^T accumulators (the MFMA's k slots of lane
//     group q are the tokens {4q..4q+3} and {16+4q..16+4q+3} of each
//     32-token block; the V^T loads use the same order). P is split into
//     bf16 hi + lo parts (two products), so the partial keeps f32-level
//     accuracy.
// 16-byte chunks of a row are stored XOR-swizzled by token so that the K
// fragment loads (16 tokens, one chunk) and the transposing V loads
// (4 tokens x 2 chunks per 16 lanes) are free of bank conflicts.

#pragma once

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

constexpr int kMaxPagesD = 512;  // pages of one partition (plus one)
constexpr float kLazyD = 8.f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

// Stored position of 16-byte chunk q (of 16) of token row t: q XOR a
// bijection of t mod 16 that maps bits (b3 b2 b1 b0) to (b3 b1 b0 b2).
// Sixteen consecutive tokens of one chunk land on sixteen positions, and the
// four tokens x two chunks of a transposing load land on eight.
__device__ __forceinline__ int dswz(int t) {
  return ((t & 3) << 1) | ((t >> 2) & 1) | (t & 8);
}

// Cache-policy operand of a global->LDS load that marks it non-temporal.
constexpr int kCachePolicyNT = 2;

// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits 3:0 and 15:14, expcnt (7) in 6:4, lgkmcnt (15) in 11:8
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The LDS of the matrix-core body, declared by the kernel that runs it: the
// ring stages (2*TT*D elements each; stages past NS are not used), each its
// own LDS object, and the partition's page ids (kMaxPagesD). Separate
// objects let the compiler's wait insertion tell the stages apart: an LDS
// read of one stage does not wait for global->LDS loads into another.
struct DmaLds {
  uint16_t* st0;
  uint16_t* st1;
  uint16_t* st2;
  uint16_t* st3;
  int* pid;
};

// The work of one workgroup of 64 * NW threads: `block` is its index in the
// grid of its launch (the decomposition below is over that index). NT: the
// K/V fetches are non-temporal (streaming) loads.
template <int D, int TT, int NS, int NW, bool SPLIT, bool NT>
__device__ __forceinline__ void partial_dma_body(const PartialArgs& a, const int block,
                                                 const DmaLds& lds) {
  constexpr int KS = D / 32;                 // k-steps of S^T
  constexpr int TB = TT / 16;                // 16-token blocks per tile
  constexpr int KB = TT / 32;                // 32-token PV steps per tile
  constexpr int DB = D / 16;                 // 16-dim output blocks
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int NI = 2 * TT * CH / 64;       // 64-lane loads per tile (K, then V)
  constexpr int NIW = NI / NW;               // ... per wave
  static_assert(CH == 16, "the swizzle covers 16 chunks per row");
  static_assert(NI % NW == 0 && TT % 32 == 0 && NS >= 2 && NS <= 4, "tile shapes");
  static_assert((NS - 2) * NIW < 64, "vmcnt range");

  uint16_t* const st0 = lds.st0;
  uint16_t* const st1 = lds.st1;
  uint16_t* const st2 = lds.st2;
  uint16_t* const st3 = lds.st3;
  int* const sm_pid = lds.pid;

  const int n_rt = (a.max_rows + 16 * NW - 1) / (16 * NW);
  int unit, rt;
  xcd_unit_tile(block, n_rt, unit, rt);
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
  const int row0 = rt * 16 * NW;
  if (row0 >= nrows) return;  // uniform

  int page0, start, end;
  part_range(a, b, p, page0, start, end);
  // causal rows: the tile loop stops at the last owned row's end; every
  // owned row sees at least the positions below end_lo (uniform)
  const int end_lo = min(end, visible_end(a, b, row0 / a.G));
  end = min(end, visible_end(a, b, (min(row0 + 16 * NW, nrows) - 1) / a.G));
  const int shift = a.p_shift;
  const int pmask = a.P - 1;
  const int pg_first = start >> shift;
  if (end > start) {
    const int n_pg = ((end - 1) >> shift) - pg_first + 1;
    for (int i = tid; i < n_pg; i += 64 * NW) {
      const int pid = a.indices[page0 + pg_first + i];
      // an id outside the pool reads row 0 (see part_range)
      sm_pid[i] = ((unsigned)pid < (unsigned)a.num_blocks) ? pid : 0;
    }
  }

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int q4 = lane >> 4;   // lane group
  const int r16 = lane & 15;  // query row within the wave / MFMA column

  // the wave's 16 query rows as B fragments: lane -> row r16, dims 32ks + 8q4 + i
  u32x4_t qf[KS];
  const int my_row = row0 + 16 * wave + r16;
  const bool live_wave = row0 + 16 * wave < nrows;  // uniform over the wave
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
    // padding rows read row 0 of request qb: always a valid address
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qb * a.Hq + head) * D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
      qf[ks] = live ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h * a.k_hstride * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + (size_t)h * a.v_hstride * 2;
  const long long kbs = a.k_bstride * 2, vbs = a.v_bstride * 2;

  auto stage = [&](int s) -> uint16_t* {
    return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3;
  };

  // Tile j -> stage s: load m (of NI) fills chunk slots [64m, 64m+64) of the
  // stage (K slots first, then V); slot c holds token c/16, stored position
  // c%16, i.e. chunk (c%16) ^ dswz(token). Rows past the end repeat the last
  // token (their scores are masked).
  auto fetch = [&](int j, uint16_t* dst) {
    const int t0 = start + j * TT;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int m = wave * NIW + i;
      const bool is_v = m >= NI / 2;
      const int mm = is_v ? m - NI / 2 : m;
      const int t = 4 * mm + (lane >> 4);
      const int q = (lane & 15) ^ dswz(t);
      const int tc = min(t0 + t, end - 1);
      const int pid = sm_pid[(tc >> shift) - pg_first];
      const char* src = (is_v ? vbase + pid * vbs : kbase + pid * kbs) + (tc & pmask) * (2 * D) + q * 16;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(dst + (is_v ? TT * D : 0) + 512 * mm),
          16, 0, NT ? kCachePolicyNT : 0);
    }
  };

  f32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float run_m = -INFINITY, run_l = 0.f;

  // per-lane LDS offsets (elements): K fragment rows 16tb + r16 with chunk
  // 4ks + q4; transposing V loads: lane group q4 of rows {4q4..4q4+3} (+16)
  // at dims 16db + 4(lane%4), lane i of the group addressing token i/4
  const int k_row = r16;
  const int k_sw = dswz(r16);
  const int v_tok = 4 * q4 + (r16 >> 2);
  const int v_sw = dswz(v_tok);            // also tokens v_tok + 16: same t mod 16
  const int v_sub = (lane & 3);            // 4-dim piece within the 16 dims
  // Each lane's V^T fragment offset (elements, within a 32-token block) for
  // the 16-dim output block db is chunk 2db + v_sub/2 of token v_tok, i.e.
  // v_base + 16 (db ^ v_w) (the swizzle's low bit only moves v_sub/2). Kept
  // to this form, a fragment address is the stage, the tile's V half, v_base,
  // the db term and a constant: few enough address steps that the compiler
  // ties every transposing load to its stage. (With one more step it loses
  // that link, and such a load waits for every global->LDS load in flight,
  // the next tiles' fetches included.)
  const int v_base = v_tok * D + 8 * ((v_sub >> 1) ^ (v_sw & 1)) + 4 * (v_sub & 1);
  const int v_w = v_sw >> 1;

  const int n_tiles = (end > start) ? (end - start + TT - 1) / TT : 0;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): query fragments have landed
  __syncthreads();                     // page ids visible
  // Every tile issues exactly one fetch, also past the last tile: such a
  // fetch reads the last token's rows (every lane the same 256 bytes of K and
  // of V) into the free stage, which nothing reads again. With a fetch on
  // every path, tile i's bytes are always followed by exactly NS - 2 later
  // fetches when tile i starts, so one constant wait count covers every
  // path; a fetch skipped on some paths makes the compiler's own wait
  // insertion assume the worst and wait for every fetch in flight.
  if (n_tiles > 0) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) fetch(j, stage(j));
  }

  auto tile = [&](int i, uint16_t* buf, uint16_t* next) {
    wait_vm<(NS - 2) * NIW>();  // tile i has landed (this wave's part)
    if (NW > 1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // every wave is past tile i - 1: its stage takes tile i + NS - 1
    fetch(i + NS - 1, next);
    // a wave without live rows only fetches and keeps the barriers
    if (!live_wave) return;
    const int t0 = start + i * TT;
    const uint16_t* kt = buf;
    const uint16_t* vt = buf + TT * D;

    // S^T = K . Q^T
    f32x4_t s[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      s[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = kt + (16 * tb + k_row) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kr + 8 * ((4 * ks + q4) ^ k_sw));
        s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), s[tb], 0, 0, 0);
      }
    }

    // row max over the lane groups (scaled log2 units)
    float cs = a.scale_log2, mx;
    if (t0 + TT <= end_lo) {
      float hi = -INFINITY, lo = INFINITY;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          hi = fmaxf(hi, s[tb][jj]);
          lo = fminf(lo, s[tb][jj]);
        }
      mx = (cs >= 0.f ? hi : lo) * cs;
    } else {
      mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = t0 + 16 * tb + 4 * q4 + jj;
          s[tb][jj] = (t < my_end) ? s[tb][jj] * cs : -INFINITY;
          mx = fmaxf(mx, s[tb][jj]);
        }
      cs = 1.f;
    }
    {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      const auto s32 = __builtin_amdgcn_permlane32_swap(f32_bits(mx), f32_bits(mx), false, false);
      mx = fmaxf(bits_f32(s32[0]), bits_f32(s32[1]));  // lanes l and l ^ 32
    }
    const int need = mx > run_m + kLazyD;
    if (__any(need)) {
      const float mn = need ? mx : run_m;
      const float corr = (mn == run_m) ? 1.f : fast_exp2(run_m - mn);
      run_l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= corr;
      run_m = mn;
    }
    const float mu = (run_m == -INFINITY) ? 0.f : run_m;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        s[tb][jj] = fast_exp2(__builtin_fmaf(s[tb][jj], cs, -mu));
        run_l += s[tb][jj];
      }

    // O^T += V^T . P^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const f32x4_t& sv = s[2 * kb + x];
        hw[2 * x] = pack_bf16x2_rne(sv[0], sv[1]);
        hw[2 * x + 1] = pack_bf16x2_rne(sv[2], sv[3]);
        if constexpr (SPLIT) {
          lw[2 * x] = pack_bf16x2_rne(sv[0] - bf16_lo(hw[2 * x]), sv[1] - bf16_hi(hw[2 * x]));
          lw[2 * x + 1] = pack_bf16x2_rne(sv[2] - bf16_lo(hw[2 * x + 1]), sv[3] - bf16_hi(hw[2 * x + 1]));
        }
      }
      const bf16x8_t ph = as_bf16x8(u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      bf16x8_t pl;
      if constexpr (SPLIT) pl = as_bf16x8(u32x4_t{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // chunk 2db + v_sub/2 of tokens 32kb + v_tok and 32kb + 16 + v_tok
        const int vo = v_base + 16 * (db ^ v_w);
        const uint16_t* p0 = vt + vo + 32 * kb * D;
        const uint16_t* p1 = vt + vo + (32 * kb + 16) * D;
        const u32x2_t v0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0));
        const u32x2_t v1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1));
        const bf16x8_t vf = as_bf16x8(u32x4_t{v0[0], v0[1], v1[0], v1[1]});
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph, acc[db], 0, 0, 0);
        if constexpr (SPLIT) acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, acc[db], 0, 0, 0);
      }
    }
  };

  // ring of NS stages: tile i computes from stage i % NS, and tile i + NS - 1
  // is fetched into the stage tile i - 1 used (free once every wave passed
  // the barrier of tile i). The loop runs whole cycles of NS tiles and the
  // last n_tiles % NS tiles follow it, each only after the one before, so
  // that every path into a tile carries the same fetches in flight (a cycle
  // cut short inside the loop would give the loop's back edge such a path).
  int i0 = 0;
  for (; i0 + NS <= n_tiles; i0 += NS) {
#pragma unroll
    for (int k = 0; k < NS; ++k) tile(i0 + k, stage(k), stage((k + NS - 1) % NS));
  }
  const int rest = n_tiles - i0;
  if (rest > 0) {
    tile(i0, stage(0), stage(NS - 1));
    if (NS > 2 && rest > 1) {
      tile(i0 + 1, stage(1), stage(0));
      if (NS > 3 && rest > 2) tile(i0 + 2, stage(2), stage(1));
    }
  }
  wait_vm<0>();  // no global->LDS load outlives the workgroup

  // row sum across the lane groups, then the normalized partial and its LSE
  float l = run_l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (my_row < nrows) {
    const int m = my_row / a.G, g = my_row % a.G;
    const size_t o = state_index(a, stacked, mbase, b, p, m, h * a.G + g);
    float* dst = a.v_out + o * D + 4 * q4;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<float4*>(dst + 16 * db) =
          make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
    if (q4 == 0) a.lse_out[o] = (l > 0.f) ? run_m + log2f(l) : -INFINITY;
  }
}

}  // namespace

}  // namespace pdk
