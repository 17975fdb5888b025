// Partition-size autotuning for cascade decode, per shape bucket, timed with
// a cold last-level cache [cascade-PR, "What I left out, and where I was
// unsure": the shape-bucketed kernel autotuner with cold-L2 benchmark
// methodology is not wired to either cascade level, which both use the
// heuristic chunk size].
//
// A tuning run builds the plan of every candidate (level-0 size x level-1
// size) on the host, uploads it to the caller's workspace, and times whole
// steps (all partial launches and the merge) on the caller's stream with HIP
// events, each timed step after a read of the caller's flush buffer that
// evicts the step's data from the last-level cache, as the rest of a model
// would between two steps of one layer. The fastest candidate is kept for
// the step's shape bucket; a later call in the same bucket returns it without
// measuring. Buckets: page size, head counts and dims, dtypes, the plan
// parameters, and powers of two (halves for the token counts) of the batch,
// the total tokens, the shared tokens and the members the plan finds.

#include <array>
#include <cmath>
#include <map>
#include <mutex>
#include <vector>

#include "device.h"
#include "internal.h"

namespace pdk {

namespace {

// Reads n16 16-byte words; the loads stay (their XOR is compared with a
// runtime value that the caller passes as one no read can produce in
// practice, and a match only writes that word back to the flush buffer).
__global__ __launch_bounds__(256) void flush_read_kernel(uint4* buf, size_t n16,
                                                         uint32_t never) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) buf[0].x = acc;
}

constexpr int kKeyLen = 16;
typedef std::array<int32_t, kKeyLen> TuneKey;

struct TuneResult {
  int32_t s0, s1;
  float us;
};

std::mutex g_tune_mu;
std::map<TuneKey, TuneResult> g_tune_cache;

int32_t log2_bucket(long long x) {  // floor(log2(x + 1))
  int32_t b = 0;
  for (unsigned long long v = (unsigned long long)(x + 1); v > 1; v >>= 1) ++b;
  return b;
}

int32_t half_log2_bucket(long long x) {  // floor(2 * log2(x + 1))
  return (int32_t)std::floor(2.0 * std::log2((double)x + 1.0));
}

int make_key(const pdk_csr* csr, int32_t P, const pdk_cascade_params* pr, const pdk_kv_pool* pool,
             int32_t Hq, int32_t q_dtype, TuneKey* key) {
  if (!csr || !pr || !pool || !key) return fail(PDK_ERR_ARG, "NULL argument");
  if (pool->num_kv_heads <= 0 || Hq <= 0 || Hq % pool->num_kv_heads)
    return fail(PDK_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq,
                pool->num_kv_heads);
  pdk_cascade_plan* plan = nullptr;
  int st = pdk_cascade_plan_create(csr, P, pr, &plan);
  if (st) return st;
  int32_t stats[6], decline = 0;
  pdk_cascade_plan_stats(plan, stats, &decline);
  pdk_cascade_plan_free(plan);
  long long tokens = 0;
  for (int b = 0; b < csr->batch; ++b) tokens += csr->kv_len[b];
  *key = TuneKey{P, pool->num_kv_heads, Hq / pool->num_kv_heads, pool->head_dim_k,
                 pool->head_dim_v, pool->dtype, q_dtype, pr->enabled,
                 pr->max_groups * 64 + pr->max_depth, pr->fuse_levels,
                 pr->min_shared_pages * 64 + pr->min_members,
                 log2_bucket(csr->batch), half_log2_bucket(tokens),
                 half_log2_bucket(stats[3]), log2_bucket(stats[1]), decline};
  return PDK_OK;
}

int check_candidates(const int32_t* c, int32_t n, int32_t P, const char* what) {
  if (!c || n <= 0) return fail(PDK_ERR_ARG, "no %s candidates", what);
  for (int i = 0; i < n; ++i)
    if (c[i] <= 0 || c[i] % P)
      return fail(PDK_ERR_ARG, "%s candidate %d is not a positive multiple of page_size %d", what,
                  c[i], P);
  return PDK_OK;
}

}  // namespace

}  // namespace pdk

using namespace pdk;

extern "C" {

int pdk_cascade_tuning_key(const pdk_csr* csr_host, int32_t page_size,
                           const pdk_cascade_params* params, const pdk_kv_pool* pool,
                           int32_t num_q_heads, int32_t q_dtype, int32_t key[16]) {
  if (!key) return fail(PDK_ERR_ARG, "NULL key");
  TuneKey k{};
  int st = make_key(csr_host, page_size, params, pool, num_q_heads, q_dtype, &k);
  if (st) return st;
  for (int i = 0; i < kKeyLen; ++i) key[i] = k[i];
  return PDK_OK;
}

void pdk_cascade_tuning_clear(void) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  g_tune_cache.clear();
}

size_t pdk_cascade_autotune_workspace_bytes(const pdk_csr* csr_host, int32_t page_size,
                                            const pdk_cascade_params* params,
                                            const int32_t* l0_candidates, int32_t n_l0,
                                            const int32_t* l1_candidates, int32_t n_l1,
                                            int32_t num_q_heads, int32_t head_dim_v) {
  if (!params || check_candidates(l0_candidates, n_l0, page_size, "level-0") ||
      check_candidates(l1_candidates, n_l1, page_size, "level-1"))
    return 0;
  size_t need = 0;
  for (int i = 0; i < n_l0; ++i)
    for (int j = 0; j < n_l1; ++j) {
      pdk_cascade_params p = *params;
      p.l0_partition_tokens = l0_candidates[i];
      p.l1_partition_tokens = l1_candidates[j];
      pdk_cascade_plan* plan = nullptr;
      if (pdk_cascade_plan_create(csr_host, page_size, &p, &plan)) return 0;
      need = std::max(need, pdk_cascade_workspace_bytes(plan, num_q_heads, head_dim_v));
      pdk_cascade_plan_free(plan);
    }
  return need;
}

int pdk_cascade_autotune(const pdk_csr* csr_host, int32_t page_size,
                         const pdk_cascade_params* params, const pdk_kv_pool* pool, const void* q,
                         int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                         const int32_t* l0_candidates, int32_t n_l0,
                         const int32_t* l1_candidates, int32_t n_l1, int32_t reps,
                         void* flush_buffer, size_t flush_bytes, void* workspace,
                         size_t workspace_bytes, float* out, float* lse_out, float* times_us,
                         hipStream_t stream, pdk_tuning* result) {
  if (!params || !pool || !q || !workspace || !out || !result)
    return fail(PDK_ERR_ARG, "NULL argument");
  int st = check_candidates(l0_candidates, n_l0, page_size, "level-0");
  if (st || (st = check_candidates(l1_candidates, n_l1, page_size, "level-1"))) return st;
  if (reps < 1) return fail(PDK_ERR_ARG, "reps %d < 1", reps);
  TuneKey key{};
  if ((st = make_key(csr_host, page_size, params, pool, num_q_heads, q_dtype, &key))) return st;
  if (times_us)
    for (int i = 0; i < n_l0 * n_l1; ++i) times_us[i] = -1.f;
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    auto it = g_tune_cache.find(key);
    if (it != g_tune_cache.end()) {
      *result = pdk_tuning{it->second.s0, it->second.s1, it->second.us, 0};
      return PDK_OK;
    }
  }
  const size_t n16 = flush_buffer ? flush_bytes / 16 : 0;
  hipEvent_t ev[2] = {nullptr, nullptr};
  if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
    if (ev[0]) (void)hipEventDestroy(ev[0]);
    return fail(PDK_ERR_HIP, "event create failed");
  }
  TuneResult best{0, 0, INFINITY};
  for (int i = 0; i < n_l0 && !st; ++i)
    for (int j = 0; j < n_l1 && !st; ++j) {
      pdk_cascade_params p = *params;
      p.l0_partition_tokens = l0_candidates[i];
      p.l1_partition_tokens = l1_candidates[j];
      pdk_cascade_plan* plan = nullptr;
      if ((st = pdk_cascade_plan_create(csr_host, page_size, &p, &plan))) break;
      st = pdk_cascade_plan_upload(plan, workspace, workspace_bytes, stream);
      double total_ms = 0.0;
      for (int r = -2; r < reps && !st; ++r) {  // two untimed runs first
        if (n16 > 0) {
          hipLaunchKernelGGL(flush_read_kernel, dim3(1024), dim3(256), 0, stream,
                             (uint4*)flush_buffer, n16, 0x9E3779B9u);
          if (hipGetLastError() != hipSuccess) { st = fail(PDK_ERR_HIP, "flush launch"); break; }
        }
        if (hipEventRecord(ev[0], stream) != hipSuccess) { st = fail(PDK_ERR_HIP, "event record"); break; }
        st = pdk_run_cascade_decode(plan, pool, q, q_dtype, num_q_heads, sm_scale, out, lse_out,
                                    workspace, workspace_bytes, stream);
        if (st) break;
        float ms = 0.f;
        if (hipEventRecord(ev[1], stream) != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
            hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) {
          st = fail(PDK_ERR_HIP, "event timing");
          break;
        }
        if (r >= 0) total_ms += ms;
      }
      // the upload read the plan's host arrays: done once the stream is idle
      if (hipStreamSynchronize(stream) != hipSuccess && !st) st = fail(PDK_ERR_HIP, "stream sync");
      pdk_cascade_plan_free(plan);
      if (st) break;
      const float us = (float)(1000.0 * total_ms / reps);
      if (times_us) times_us[i * n_l1 + j] = us;
      if (us < best.us) best = TuneResult{p.l0_partition_tokens, p.l1_partition_tokens, us};
    }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (st) return st;
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tune_cache[key] = best;
  }
  *result = pdk_tuning{best.s0, best.s1, best.us, 1};
  return PDK_OK;
}

int pdk_cascade_tuned_params(const pdk_csr* csr_host, int32_t page_size,
                             const pdk_cascade_params* params, const pdk_kv_pool* pool,
                             int32_t num_q_heads, int32_t q_dtype, pdk_cascade_params* tuned,
                             int32_t* found) {
  if (!tuned || !found) return fail(PDK_ERR_ARG, "NULL argument");
  TuneKey key{};
  int st = make_key(csr_host, page_size, params, pool, num_q_heads, q_dtype, &key);
  if (st) return st;
  *tuned = *params;
  *found = 0;
  std::lock_guard<std::mutex> lock(g_tune_mu);
  auto it = g_tune_cache.find(key);
  if (it != g_tune_cache.end()) {
    tuned->l0_partition_tokens = it->second.s0;
    tuned->l1_partition_tokens = it->second.s1;
    *found = 1;
  }
  return PDK_OK;
}

}  // extern "C"
