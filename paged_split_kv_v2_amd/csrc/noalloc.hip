// Flat split-KV decode that allocates nothing: pdk_decode_flat with its
// partial states in a file-scope device array instead of a caller
// workspace, for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is one per device (each GPU the library runs on holds its own
// copy until the process ends). Host code never names it except to look
// up its device address: hipGetSymbolAddress, once per device with that
// device current, and that address is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "pdk.h"

namespace {

constexpr size_t kScratchBytes = PDK_DECODE_FLAT_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pdk::fail(PDK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pdk::fail(PDK_ERR_UNSUPPORTED, "device %d outside the %d devices served", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pdk::fail(PDK_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PDK_OK;
}

}  // namespace

extern "C" int pdk_decode_flat_noalloc(const pdk_kv_pool* pool, const pdk_csr* csr_dev,
                                       const void* q, int32_t q_dtype, int32_t num_q_heads,
                                       float sm_scale, int32_t partition_tokens,
                                       const int32_t* part_indptr_dev, int32_t num_partitions,
                                       float* out, float* lse_out, hipStream_t stream) {
  if (!pool) return pdk::fail(PDK_ERR_ARG, "pool is NULL");
  if (num_partitions < 0 || num_q_heads <= 0 || pool->head_dim_v <= 0)
    return pdk::fail(PDK_ERR_ARG, "num_partitions %d, num_q_heads %d, head_dim_v %d",
                     num_partitions, num_q_heads, pool->head_dim_v);
  const size_t need = pdk_decode_flat_workspace_bytes(num_partitions, num_q_heads,
                                                      pool->head_dim_v);
  if (need > kScratchBytes)
    return pdk::fail(PDK_ERR_WORKSPACE,
                     "partial states of %d partitions x %d heads x %d dims need %zu bytes, "
                     "more than the %zu-byte static scratch of pdk_decode_flat_noalloc",
                     num_partitions, num_q_heads, pool->head_dim_v, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st) return st;
  }
  // every state row the merge reads is written by this call's partial
  // launch, so nothing left in the array by an earlier call is read
  return pdk_decode_flat(pool, csr_dev, q, q_dtype, num_q_heads, sm_scale, partition_tokens,
                         part_indptr_dev, num_partitions, out, lse_out, ws,
                         need > 0 ? kScratchBytes : 0, stream);
}
