// Host side of the C ABI: argument checks, partition bookkeeping, the
// shared-prefix planner, the chunked-prefix plan, and launch orchestration.
//
// Sources: [cascade-PR] mlxcel pull request "perf(core): compute shared
// prompt prefixes once per decode batch"; [DCP-PR] ROCm/ATOM pull request
// "[feat][DCP] Optimize MLA DCP (Enable Prefix Cache / Chunked Prefill + FP8
// KVCache)". Each function names the section it follows.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "internal.h"
#include "pdk.h"

namespace pdk {

static thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}


static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int pshift(int P) {
  if (P <= 0 || (P & (P - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < P) ++s;
  return s;
}

// Checks shared by every entry point that reads a pool.
static int check_pool(const pdk_kv_pool* pool) {
  if (!pool || !pool->k) return fail(PDK_ERR_ARG, "pool or pool->k is NULL");
  if (pool->num_blocks <= 0 || pool->page_size <= 0 || pool->num_kv_heads <= 0 ||
      pool->head_dim_k <= 0 || pool->head_dim_v <= 0)
    return fail(PDK_ERR_ARG, "pool sizes must be positive");
  if (pool->dtype != PDK_F32 && pool->dtype != PDK_BF16 && pool->dtype != PDK_FP8_E4M3)
    return fail(PDK_ERR_DTYPE, "unknown pool dtype %d", pool->dtype);
  if (!pool->v && pool->head_dim_v > pool->head_dim_k)
    return fail(PDK_ERR_SHAPE, "latent pool: head_dim_v %d > head_dim_k %d", pool->head_dim_v,
                pool->head_dim_k);
  if (!aligned16(pool->k) || (pool->v && !aligned16(pool->v)))
    return fail(PDK_ERR_ARG, "pool base pointers must be 16-byte aligned");
  return PDK_OK;
}

static void fill_pool_args(const pdk_kv_pool* pool, PartialArgs& a) {
  a.k = pool->k;
  a.v = pool->v;
  a.num_blocks = pool->num_blocks;
  a.P = pool->page_size;
  a.p_shift = pshift(pool->page_size);
  a.Hkv = pool->num_kv_heads;
  a.Dk = pool->head_dim_k;
  a.Dv = pool->head_dim_v;
  a.kv_dtype = pool->dtype;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.k_hstride = (long long)pool->page_size * pool->head_dim_k;
  a.k_bstride = a.k_hstride * pool->num_kv_heads;
  a.v_hstride = (long long)pool->page_size * (pool->v ? pool->head_dim_v : pool->head_dim_k);
  a.v_bstride = a.v_hstride * pool->num_kv_heads;
}

static int check_query(const void* q, int q_dtype, int Hq, const pdk_kv_pool* pool) {
  if (!q) return fail(PDK_ERR_ARG, "q is NULL");
  if (q_dtype != PDK_F32 && q_dtype != PDK_BF16)
    return fail(PDK_ERR_DTYPE, "q dtype must be f32 or bf16 (got %d)", q_dtype);
  if (Hq <= 0 || Hq % pool->num_kv_heads != 0)
    return fail(PDK_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d", Hq,
                pool->num_kv_heads);
  return PDK_OK;
}

int partial_args(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q, int q_dtype, int Hq,
                 float sm_scale, int S, const int* part_indptr, int num_parts,
                 const int* member_indptr, const int* members, int max_members, int G,
                 const int* out_row_base, float* v_out, float* lse_out, const int2* work,
                 PartialArgs* out, bool* empty, int q_tokens, int causal) {
  *empty = true;
  int st = check_pool(pool);
  if (st) return st;
  if ((st = check_query(q, q_dtype, Hq, pool))) return st;
  if (!csr || csr->batch < 0 || csr->nnz < 0)
    return fail(PDK_ERR_ARG, "csr is NULL, batch < 0 or nnz < 0");
  if (S <= 0 || S % pool->page_size != 0)
    return fail(PDK_ERR_ARG, "partition_tokens %d must be a positive multiple of page_size %d", S,
                pool->page_size);
  if (num_parts < 0) return fail(PDK_ERR_ARG, "num_partitions < 0");
  if (num_parts == 0 || csr->batch == 0) return PDK_OK;
  if (!csr->indptr || !csr->indices || !csr->kv_len || !part_indptr || !v_out || !lse_out ||
      !out_row_base)
    return fail(PDK_ERR_ARG, "NULL device array");
  if (member_indptr && (!members || max_members <= 0))
    return fail(PDK_ERR_ARG, "stacked view without members");
  if (q_tokens < 1 || (causal != 0 && causal != 1))
    return fail(PDK_ERR_ARG, "q_tokens %d must be >= 1 and causal 0 or 1", q_tokens);
  if (causal && member_indptr)
    return fail(PDK_ERR_UNSUPPORTED, "causal masking is for flat views only");
  if (!aligned16(q) || !aligned16(v_out)) return fail(PDK_ERR_ARG, "q/v_part must be 16-byte aligned");
  PartialArgs a{};
  fill_pool_args(pool, a);
  a.indptr = csr->indptr;
  a.indices = csr->indices;
  a.kv_len = csr->kv_len;
  a.batch = csr->batch;
  a.nnz = csr->nnz;
  a.part_indptr = part_indptr;
  a.num_parts = num_parts;
  a.S = S;
  a.q = q;
  a.q_dtype = q_dtype;
  a.Hq = Hq;
  a.G = G;
  a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.member_indptr = member_indptr;
  a.members = members;
  a.q_tokens = q_tokens;
  a.causal = causal;
  a.max_rows = (member_indptr ? max_members : 1) * q_tokens * G;
  a.out_row_base = out_row_base;
  a.v_out = v_out;
  a.lse_out = lse_out;
  a.work = work;
  *out = a;
  *empty = false;
  return PDK_OK;
}

int partial_rows(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q, int q_dtype, int Hq,
                 float sm_scale, int S, const int* part_indptr, int num_parts,
                 const int* member_indptr, const int* members, int max_members, int G,
                 const int* out_row_base, float* v_out, float* lse_out, hipStream_t stream,
                 const int2* work, int q_tokens, int causal) {
  PartialArgs a{};
  bool empty = true;
  int st = partial_args(pool, csr, q, q_dtype, Hq, sm_scale, S, part_indptr, num_parts,
                        member_indptr, members, max_members, G, out_row_base, v_out, lse_out,
                        work, &a, &empty, q_tokens, causal);
  if (st || empty) return st;
  return launch_partial(a, stream);
}

int merge_rows(const float* v_in, const float* lse_in, int num_in, const int* o_indptr,
               int num_out, int H, int D, float* v_out, float* lse_out, int out_stride,
               hipStream_t stream) {
  if (num_out < 0 || num_in < 0 || H <= 0 || D <= 0 || out_stride < 1)
    return fail(PDK_ERR_ARG, "bad merge sizes");
  if (D % 4 != 0) return fail(PDK_ERR_SHAPE, "head_dim %d is not a multiple of 4", D);
  if (num_out == 0) return PDK_OK;
  if ((num_in > 0 && (!v_in || !lse_in)) || !o_indptr || !v_out)
    return fail(PDK_ERR_ARG, "NULL merge array");
  if (!aligned16(v_in) || !aligned16(v_out)) return fail(PDK_ERR_ARG, "v_in/v_out must be 16-byte aligned");
  return launch_merge(v_in, lse_in, num_in, o_indptr, num_out, H, D, v_out, lse_out, out_stride,
                      stream);
}

// Kernel choice for one partial launch: the matrix-core paths for bf16
// queries when a KV head serves at least 16 query rows (head dim 128 with
// bf16 K/V; more than 16 on small pages) or at least 64 (MLA latent rows),
// where the products are dense 16-row tiles; otherwise the vector path,
// which keeps up to 16 query rows per KV head in registers and tiles more
// rows over several workgroups.
int launch_partial(const PartialArgs& a, hipStream_t stream) {
  bool handled = false;
  int st = launch_partial_latent(a, stream, &handled);
  if (st || handled) return st;
  st = launch_partial_dma(a, stream, &handled);
  if (st || handled) return st;
  st = launch_partial_mfma(a, stream, &handled);
  if (st || handled) return st;
  if (a.kv_dtype == PDK_FP8_E4M3)
    return fail(PDK_ERR_UNSUPPORTED, "fp8 pools are read by the matrix-core path only "
                                     "(bf16 queries, >= 64 query rows, head dims 576/512)");
  return launch_partial_valu(a, stream);
}

}  // namespace pdk

using namespace pdk;

extern "C" {

const char* pdk_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// Host-side integer work
// ---------------------------------------------------------------------------

int pdk_partition_indptr(const int32_t* kv_len, int32_t batch, int32_t partition_tokens,
                         int32_t* part_indptr) {
  if (!part_indptr || (batch > 0 && !kv_len)) return fail(PDK_ERR_ARG, "NULL argument");
  if (batch < 0) return fail(PDK_ERR_ARG, "batch %d < 0", batch);
  if (partition_tokens <= 0) return fail(PDK_ERR_ARG, "partition_tokens %d <= 0", partition_tokens);
  long long acc = 0;
  part_indptr[0] = 0;
  for (int b = 0; b < batch; ++b) {
    if (kv_len[b] < 0) return fail(PDK_ERR_ARG, "kv_len[%d] = %d < 0", b, kv_len[b]);
    acc += ceil_div(kv_len[b], partition_tokens);
    if (acc > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "too many partitions");
    part_indptr[b + 1] = (int32_t)acc;
  }
  return PDK_OK;
}

int pdk_validate_csr(const pdk_csr* csr, int32_t page_size, int32_t num_blocks) {
  if (!csr || !csr->indptr || (csr->batch > 0 && !csr->kv_len) || (csr->nnz > 0 && !csr->indices))
    return fail(PDK_ERR_ARG, "NULL page-table array");
  if (page_size <= 0 || num_blocks < 0 || csr->batch < 0)
    return fail(PDK_ERR_ARG, "bad page_size/num_blocks/batch");
  if (csr->indptr[0] != 0) return fail(PDK_ERR_SHAPE, "indptr[0] = %d != 0", csr->indptr[0]);
  for (int b = 0; b < csr->batch; ++b) {
    const int n = csr->indptr[b + 1] - csr->indptr[b];
    if (n < 0) return fail(PDK_ERR_SHAPE, "indptr decreases at %d", b);
    if (csr->kv_len[b] < 0) return fail(PDK_ERR_SHAPE, "kv_len[%d] < 0", b);
    if (n != ceil_div(csr->kv_len[b], page_size))
      return fail(PDK_ERR_SHAPE, "request %d: %d pages for %d tokens at page size %d", b, n,
                  csr->kv_len[b], page_size);
  }
  if (csr->indptr[csr->batch] != csr->nnz)
    return fail(PDK_ERR_SHAPE, "indptr[batch] = %d != nnz %d", csr->indptr[csr->batch], csr->nnz);
  for (int i = 0; i < csr->nnz; ++i)
    if (csr->indices[i] < 0 || csr->indices[i] >= num_blocks)
      return fail(PDK_ERR_SHAPE, "indices[%d] = %d outside [0, %d)", i, csr->indices[i], num_blocks);
  return PDK_OK;
}

int pdk_parse_switch(const char* value) {
  if (!value) return -1;
  std::string s(value);
  size_t a = 0, e = s.size();
  while (a < e && std::isspace((unsigned char)s[a])) ++a;
  while (e > a && std::isspace((unsigned char)s[e - 1])) --e;
  s = s.substr(a, e - a);
  for (auto& c : s) c = (char)std::tolower((unsigned char)c);
  if (s == "0" || s == "false" || s == "off" || s == "no") return 0;
  if (s == "1" || s == "true" || s == "on" || s == "yes") return 1;
  return -1;
}

int pdk_cascade_enabled_from_env(const char* var_name) {
  if (!var_name) return -1;
  return pdk_parse_switch(std::getenv(var_name));
}

int pdk_stacked_head_map(int32_t M, int32_t Hkv, int32_t G, int32_t* out) {
  if (!out || M < 0 || Hkv <= 0 || G <= 0) return fail(PDK_ERR_ARG, "bad head-map arguments");
  const int Hq = Hkv * G;
  for (int kv = 0; kv < Hkv; ++kv)
    for (int m = 0; m < M; ++m)
      for (int g = 0; g < G; ++g) out[kv * (M * G) + m * G + g] = m * Hq + kv * G + g;
  return PDK_OK;
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

int pdk_paged_decode_partial(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q,
                             int32_t q_dtype, int32_t Hq, float sm_scale, int32_t S,
                             const int32_t* part_indptr, int32_t num_parts, float* v_part,
                             float* lse_part, hipStream_t stream) {
  int st = check_pool(pool);
  if (st) return st;
  if ((st = check_query(q, q_dtype, Hq, pool))) return st;
  return partial_rows(pool, csr, q, q_dtype, Hq, sm_scale, S, part_indptr, num_parts, nullptr,
                      nullptr, 0, Hq / pool->num_kv_heads, part_indptr, v_part, lse_part, stream);
}

int pdk_paged_multi_token_partial(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q,
                                  int32_t q_dtype, int32_t Hq, int32_t T, int32_t causal,
                                  float sm_scale, int32_t S, const int32_t* part_indptr,
                                  int32_t num_parts, float* v_part, float* lse_part,
                                  hipStream_t stream) {
  int st = check_pool(pool);
  if (st) return st;
  if ((st = check_query(q, q_dtype, Hq, pool))) return st;
  return partial_rows(pool, csr, q, q_dtype, Hq, sm_scale, S, part_indptr, num_parts, nullptr,
                      nullptr, 0, Hq / pool->num_kv_heads, part_indptr, v_part, lse_part, stream,
                      nullptr, T, causal);
}

int pdk_multi_token_flat(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q,
                         int32_t q_dtype, int32_t Hq, int32_t T, int32_t causal, float sm_scale,
                         int32_t S, const int32_t* part_indptr, int32_t num_parts, float* out,
                         float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_pool(pool);
  if (st) return st;
  if (!csr || !out) return fail(PDK_ERR_ARG, "NULL csr/out");
  if (T < 1 || Hq <= 0 || (long long)T * Hq > 0x7FFFFFFF)
    return fail(PDK_ERR_ARG, "q_tokens %d, num_q_heads %d", T, Hq);
  const int H = T * Hq;  // (token, head) pairs merge as heads
  const size_t need = pdk_decode_flat_workspace_bytes(num_parts, H, pool->head_dim_v);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  float* v_part = (float*)ws;
  float* lse_part = (float*)((char*)ws + (((size_t)num_parts * H * pool->head_dim_v * 4 + 255) & ~(size_t)255));
  if (num_parts > 0) {
    st = pdk_paged_multi_token_partial(pool, csr, q, q_dtype, Hq, T, causal, sm_scale, S,
                                       part_indptr, num_parts, v_part, lse_part, stream);
    if (st) return st;
  }
  return pdk_merge_states(v_part, lse_part, num_parts, part_indptr, csr->batch, H,
                          pool->head_dim_v, out, lse_out, stream);
}

int pdk_merge_states(const float* v_in, const float* lse_in, int32_t num_in,
                     const int32_t* o_indptr, int32_t num_out, int32_t H, int32_t D, float* v_out,
                     float* lse_out, hipStream_t stream) {
  return merge_rows(v_in, lse_in, num_in, o_indptr, num_out, H, D, v_out, lse_out, 1, stream);
}

size_t pdk_decode_flat_workspace_bytes(int32_t num_parts, int32_t Hq, int32_t Dv) {
  if (num_parts <= 0 || Hq <= 0 || Dv <= 0) return 0;
  const size_t rows = (size_t)num_parts * Hq;
  return ((rows * Dv * sizeof(float) + 255) & ~(size_t)255) + rows * sizeof(float);
}

int pdk_decode_flat(const pdk_kv_pool* pool, const pdk_csr* csr, const void* q, int32_t q_dtype,
                    int32_t Hq, float sm_scale, int32_t S, const int32_t* part_indptr,
                    int32_t num_parts, float* out, float* lse_out, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_pool(pool);
  if (st) return st;
  if (!csr || !out) return fail(PDK_ERR_ARG, "NULL csr/out");
  const size_t need = pdk_decode_flat_workspace_bytes(num_parts, Hq, pool->head_dim_v);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(PDK_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  float* v_part = (float*)ws;
  float* lse_part = (float*)((char*)ws + (((size_t)num_parts * Hq * pool->head_dim_v * 4 + 255) & ~(size_t)255));
  if (num_parts > 0) {
    st = pdk_paged_decode_partial(pool, csr, q, q_dtype, Hq, sm_scale, S, part_indptr, num_parts,
                                  v_part, lse_part, stream);
    if (st) return st;
  }
  return pdk_merge_states(v_part, lse_part, num_parts, part_indptr, csr->batch, Hq,
                          pool->head_dim_v, out, lse_out, stream);
}

int pdk_stack_heads(const void* q, int32_t q_dtype, const int32_t* members, int32_t M,
                    int32_t Hkv, int32_t G, int32_t D, void* q0, hipStream_t stream) {
  if (M < 0 || Hkv <= 0 || G <= 0 || D <= 0) return fail(PDK_ERR_ARG, "bad stack sizes");
  if (q_dtype != PDK_F32 && q_dtype != PDK_BF16) return fail(PDK_ERR_DTYPE, "q dtype %d", q_dtype);
  if (M == 0) return PDK_OK;
  if (!q || !members || !q0) return fail(PDK_ERR_ARG, "NULL stack array");
  return launch_stack(q, q_dtype, members, M, Hkv, G, D, q0, stream);
}

int pdk_unstack_heads(const float* v0, const float* lse0, int32_t M, int32_t Hkv, int32_t G,
                      int32_t D, float* v_out, float* lse_out, hipStream_t stream) {
  if (M < 0 || Hkv <= 0 || G <= 0 || D <= 0) return fail(PDK_ERR_ARG, "bad unstack sizes");
  if (M == 0) return PDK_OK;
  if (!v0 || !v_out || (!lse0) != (!lse_out)) return fail(PDK_ERR_ARG, "NULL unstack array");
  return launch_unstack(v0, lse0, M, Hkv, G, D, v_out, lse_out, stream);
}

int pdk_fp8_dequant_bf16(const uint8_t* in, int64_t n, float scale, uint16_t* out,
                         hipStream_t stream) {
  if (n < 0) return fail(PDK_ERR_ARG, "n < 0");
  if (n == 0) return PDK_OK;
  if (!in || !out) return fail(PDK_ERR_ARG, "NULL dequant array");
  return launch_dequant(in, n, scale, out, stream);
}

}  // extern "C"
