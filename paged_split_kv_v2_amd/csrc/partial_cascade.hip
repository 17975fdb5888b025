// Both levels of a cascade step in one launch [cascade-PR = mlxcel pull
// request "perf(core): compute shared prompt prefixes once per decode
// batch", section "The decomposition, and the one part that is not
// obvious": level 0 reads each shared span once for the members' stacked
// query rows, level 1 reads every request's own remaining pages; the two
// write disjoint partial rows, so neither depends on the other].
//
// Run back to back, level 0 (a few hundred long workgroups, one per
// (group, partition, KV head)) leaves most of the chip idle while it drains
// and level 1 waits for it. One grid holds both: its first blocks0 blocks
// run the level-0 body (matrix cores, LDS-ring staging), the rest run the
// level-1 body (vector ALU), so level-1 workgroups fill the compute units
// beside the level-0 ones. The bodies are the same functions the
// single-level kernels run, so every partial row is bit-identical to the one
// the two separate launches write.

#include "partial_dma_body.h"
#include "partial_valu_body.h"

namespace pdk {

namespace {

constexpr int kL0Waves = 4;  // level-0 body: 4 waves x 16 stacked query rows
constexpr int kL0Stages = 2;  // level-0 LDS ring: two 32-token stages
// Level-0 rows with non-temporal (streaming) loads, like level 1. Timed on
// the step a model sees, after a read that evicts the last-level cache
// (other layers run between two steps of one layer), the 72-request
// shared-prefix step takes 65.7 us with them against 68.0 us with cached
// level-0 loads; only when steps of one layer run back to back, so that the
// step's 0.28 GB of unique bytes partly stay in the 256 MB last-level
// cache, do cached loads win (58.6 against 61.9 us).
constexpr bool kL0Streaming = true;
static_assert(64 * kL0Waves == kThreads, "both bodies run on 256-thread workgroups");

// Three workgroups per compute unit: the level-1 body alone fits three (156
// registers), and with a two-stage ring the level-0 body keeps its
// accumulators in the same budget (160 registers, no accumulator registers).
// The level-1 body's LDS (the cross-wave merge and its page ids) overlays the
// first ring stage, since no workgroup runs both bodies: 34 KB per
// workgroup. A three-stage ring then also fits three workgroups (50 KB), but
// measured on the batch-72 shared-prefix step it is no faster (62.5 against
// 61.0 us per cold step): alone in the grid, level 0 takes 33 us and level 1
// 42 us, so the level-1 workgroups, which hold most of the bytes, set the
// pace, not the level-0 ring's depth.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void cascade_partial_kernel(const PartialArgs a0, const PartialArgs a1, const int blocks0) {
  constexpr int kStage = 2 * 32 * 128;  // one K + V tile of 32 tokens (bf16 elements)
  __shared__ __align__(16) uint16_t st0[kStage];
  __shared__ __align__(16) uint16_t st1[kStage];
  __shared__ __align__(16) uint16_t st2[kL0Stages > 2 ? kStage : 8];
  __shared__ __align__(16) uint16_t st3[kL0Stages > 3 ? kStage : 8];
  __shared__ int pid0[kMaxPagesD];
  using L1Lds = ValuLds<4, 128>;
  static_assert(sizeof(L1Lds) <= sizeof(st0), "level-1 LDS overlays the first ring stage");
  const int bid = blockIdx.x;
  if (bid < blocks0)
    partial_dma_body<128, 32, kL0Stages, kL0Waves, true, kL0Streaming>(
        a0, bid, DmaLds{st0, st1, st2, st3, pid0});
  else  // a level-1 workgroup never runs the level-0 body: its LDS is free
    partial_valu_body<KV_BF16, PDK_BF16, 128, 4, true, false>(
        a1, bid - blocks0, *reinterpret_cast<L1Lds*>(st0));
}

}  // namespace

// The fused launch covers bf16 K/V pools of head dim 128 with bf16 queries,
// pages of a power of two >= 16 tokens, level 0 on the matrix-core body
// (at least 16 stacked rows per KV head, as for its own launch) and level 1
// on the vector body with a row tile of 4 query rows (3 or 4 rows per KV
// head). Any other shape is left to the separate launches (*handled false).
// (A row tile of 8 would need more registers than three workgroups per
// compute unit leave.)
int launch_cascade_partials(const PartialArgs& a0, const PartialArgs& a1, hipStream_t stream,
                            bool* handled) {
  *handled = false;
  auto bf16_d128 = [](const PartialArgs& a) {
    return a.q_dtype == PDK_BF16 && a.kv_dtype == PDK_BF16 && a.v != nullptr && a.Dk == 128 &&
           a.Dv == 128 && a.p_shift >= 4;
  };
  if (!bf16_d128(a0) || !bf16_d128(a1) || a0.max_rows < 16 || a1.member_indptr != nullptr ||
      a0.q_tokens != 1 || a1.q_tokens != 1)
    return PDK_OK;
  if (a0.S / a0.P + 1 > kMaxPagesD || a1.S / a1.P + 1 > kMaxPartPages) return PDK_OK;
  // the row tile the level-1 launch of its own would take (vector launcher)
  int gm = 1;
  while (gm < a1.max_rows && gm < valu_max_rows(a1.Dk)) gm <<= 1;
  if (gm != 4) return PDK_OK;
  const long long blocks0 = xcd_grid_blocks(
      (long long)a0.num_parts * a0.Hkv, (a0.max_rows + 16 * kL0Waves - 1) / (16 * kL0Waves));
  const long long blocks1 = (long long)a1.num_parts * a1.Hkv;  // one row tile
  if (blocks0 == 0 || blocks1 == 0) return PDK_OK;
  if (blocks0 + blocks1 > 0x7FFFFFFFLL)
    return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks0 + blocks1);
  *handled = true;
  hipLaunchKernelGGL(cascade_partial_kernel, dim3((unsigned)(blocks0 + blocks1)), dim3(256), 0,
                     stream, a0, a1, (int)blocks0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(PDK_ERR_HIP, "cascade partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
