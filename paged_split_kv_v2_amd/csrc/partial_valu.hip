// Paged split-KV partial attention, vector-ALU path: kernel instantiations
// and their launcher. The per-workgroup computation is partial_valu_body
// (partial_valu_body.h), shared with the cascade kernel.

#include "partial_valu_body.h"

namespace pdk {

namespace {

template <int KT, int QT, int D, int GM, bool UNIF, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void partial_valu_kernel(const PartialArgs a) {
  __shared__ ValuLds<GM, D> lds;
  partial_valu_body<KT, QT, D, GM, UNIF, CAUSAL>(a, blockIdx.x, lds);
}

typedef void (*KernelFn)(const PartialArgs);

template <int KT, int QT, int D, bool U, bool C>
KernelFn pick_gm(int gm) {
  constexpr int E = D / 16;
  switch (gm) {
    case 1: return partial_valu_kernel<KT, QT, D, 1, U, C>;
    case 2: return partial_valu_kernel<KT, QT, D, 2, U, C>;
    case 4: return partial_valu_kernel<KT, QT, D, 4, U, C>;
    case 8: if constexpr (8 * E <= 128) return partial_valu_kernel<KT, QT, D, 8, U, C>; else return nullptr;
    case 16: if constexpr (16 * E <= 128) return partial_valu_kernel<KT, QT, D, 16, U, C>; else return nullptr;
  }
  return nullptr;
}

template <int KT, int QT, int D>
KernelFn pick_uc(int gm, bool unif, bool causal) {
  if (causal) return unif ? pick_gm<KT, QT, D, true, true>(gm) : pick_gm<KT, QT, D, false, true>(gm);
  return unif ? pick_gm<KT, QT, D, true, false>(gm) : pick_gm<KT, QT, D, false, false>(gm);
}

template <int KT, int QT>
KernelFn pick_d(int d, int gm, bool unif, bool causal) {
  switch (d) {
    case 64: return pick_uc<KT, QT, 64>(gm, unif, causal);
    case 128: return pick_uc<KT, QT, 128>(gm, unif, causal);
    case 256: return pick_uc<KT, QT, 256>(gm, unif, causal);
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
  if (a.p_shift < 0)
    return fail(PDK_ERR_UNSUPPORTED, "vector path needs a power-of-two page size (got %d)", a.P);
  if (a.S / a.P + 1 > kMaxPartPages)
    return fail(PDK_ERR_UNSUPPORTED, "partition of %d tokens spans more than %d pages", a.S,
                kMaxPartPages - 1);
  int gm = 1;
  while (gm < a.max_rows && gm < valu_max_rows(a.Dk)) gm <<= 1;
  KernelFn fn = nullptr;
  const int kt = a.kv_dtype, qt = a.q_dtype;
  const bool unif = a.P >= 16;  // a wave's four tokens of one step share a page
  // one token per request sees its whole range: the causal mask is a no-op
  const bool causal = a.causal && a.q_tokens > 1;
  if (kt == PDK_F32 && qt == PDK_F32) fn = pick_d<KV_F32, PDK_F32>(a.Dk, gm, unif, causal);
  else if (kt == PDK_F32 && qt == PDK_BF16) fn = pick_d<KV_F32, PDK_BF16>(a.Dk, gm, unif, causal);
  else if (kt == PDK_BF16 && qt == PDK_F32) fn = pick_d<KV_BF16, PDK_F32>(a.Dk, gm, unif, causal);
  else if (kt == PDK_BF16 && qt == PDK_BF16) fn = pick_d<KV_BF16, PDK_BF16>(a.Dk, gm, unif, causal);
  if (!fn)
    return fail(PDK_ERR_UNSUPPORTED,
                "no vector kernel for kv dtype %d, q dtype %d, head dim %d, %d rows", kt, qt,
                a.Dk, gm);
  const int n_tiles = (a.max_rows + gm - 1) / gm;
  const long long blocks = xcd_grid_blocks((long long)a.num_parts * a.Hkv, n_tiles);
  if (blocks == 0) return PDK_OK;
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "grid too large (%lld)", blocks);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "partial launch: %s", hipGetErrorString(err));
  return PDK_OK;
}

}  // namespace pdk
