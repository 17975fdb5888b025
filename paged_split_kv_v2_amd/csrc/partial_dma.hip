// Paged split-KV partial attention for bf16 K/V pools of head dim 128 on
// the matrix cores with global->LDS staging: kernel instantiation and its
// launcher. The per-workgroup computation is partial_dma_body
// (partial_dma_body.h), shared with the cascade kernel.

#include "partial_dma_body.h"

namespace pdk {

namespace {

// Three workgroups per compute unit, each with a three-stage ring (160
// registers, accumulators included, and 50 KB of LDS): two tiles are in
// flight while one is multiplied. Measured on the 4-token Llama-3-8B step
// (16 rows per KV head): 217 us, against 221 us for a two-stage ring at four
// workgroups per compute unit (128 registers, one spilled) or at three.
//
// The K/V rows are fetched with non-temporal loads, as the vector kernel reads
// them: 4-token Llama-3-8B step 233 -> 220 us (1.2 GB, far more than the
// last-level cache holds, so caching them only evicts other data).
template <int D, int TT, int NS, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3, 3)))
void partial_dma_kernel(const PartialArgs a) {
  __shared__ __align__(16) uint16_t st0[2 * TT * D];
  __shared__ __align__(16) uint16_t st1[2 * TT * D];
  __shared__ __align__(16) uint16_t st2[(NS > 2) ? 2 * TT * D : 8];
  __shared__ __align__(16) uint16_t st3[(NS > 3) ? 2 * TT * D : 8];
  __shared__ int pid[kMaxPagesD];
  partial_dma_body<D, TT, NS, NW, SPLIT, true>(a, blockIdx.x, DmaLds{st0, st1, st2, st3, pid});
}

typedef void (*DmaFn)(const PartialArgs);

}  // namespace

// bf16 K/V pools of head dim 128 (separate K and V), bf16 queries, pages of
// a power of two >= 4 tokens, at least 16 query rows per KV head (stacked
// level-0 rows, multi-token steps, query groups of 16): this path takes the
// launch (*handled) with 4 waves (64 rows per row tile). Below 16 rows a
// 16-row product tile would be partly padding - not a dense contraction -
// and the vector kernel takes the launch.
int launch_partial_dma(const PartialArgs& a, hipStream_t stream, bool* handled) {
  *handled = false;
  if (a.q_dtype != PDK_BF16 || a.kv_dtype != PDK_BF16 || a.v == nullptr || a.Dk != 128 ||
      a.Dv != 128 || a.p_shift < 2 || a.max_rows < 16)
    return PDK_OK;
  const int nw = 4;
  DmaFn fn = partial_dma_kernel<128, 32, 3, 4, true>;
  if (a.S / a.P + 1 > kMaxPagesD)
    return fail(PDK_ERR_UNSUPPORTED, "partition of %d tokens spans more than %d pages", a.S,
                kMaxPagesD - 1);
  *handled = true;
  const int n_rt = (a.max_rows + 16 * nw - 1) / (16 * nw);
  const long long blocks = xcd_grid_blocks((long long)a.num_parts * a.Hkv, n_rt);
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * nw), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "dma partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
