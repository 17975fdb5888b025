/*
 * pdk.h - paged split-KV decode attention for MI355X (gfx950): C ABI.
 *
 * Sources, cited by page title and section:
 *   [cascade-PR]  mlxcel pull request "perf(core): compute shared prompt
 *                 prefixes once per decode batch".
 *   [DCP-PR]      ROCm/ATOM pull request "[feat][DCP] Optimize MLA DCP
 *                 (Enable Prefix Cache / Chunked Prefill + FP8 KVCache)".
 *   [OCP-FP8]     OCP 8-bit floating point specification (E4M3).
 *
 * Conventions for every entry point:
 *   - Return value is a pdk_status; PDK_OK (0) on success. Nothing aborts or
 *     throws across this boundary. pdk_last_error() returns a thread-local
 *     message describing the last non-OK status on the calling thread.
 *   - GPU work is enqueued asynchronously on the given hipStream_t (0 = the
 *     null stream). No entry point allocates device memory: the caller owns
 *     every buffer, and workspaces are sized by the *_workspace_bytes queries.
 *   - Pointers named *_dev or documented "device" are device pointers; all
 *     others are host pointers. Device pointers are borrowed for the call
 *     (and until the enqueued work has finished); the library keeps none.
 *   - State tensors: partial and merged outputs are float32, normalized by
 *     their own softmax denominator; LSEs are float32 in log2 units,
 *     lse = m + log2(l) where m is the running max of the log2-scaled scores
 *     and l the sum of 2^(s - m) [cascade-PR, "How the #898 merge kernel is
 *     reused"]. An empty key range yields out = 0, lse = -inf.
 *   - KV pools are HND: [num_blocks, num_kv_heads, page_size, head_dim], row
 *     major. A latent pool (MLA) has one KV head, v == NULL and
 *     head_dim_v <= head_dim_k: the value of a token is the first head_dim_v
 *     lanes of its key row [DCP-PR, 3.2: the compressed latent serves as both].
 *   - Page table: CSR indptr[batch+1], indices[indptr[batch]] (pool rows),
 *     kv_len[batch] (tokens). Token t of request b lives in slot t % P of row
 *     indices[indptr[b] + t / P]; indptr[b+1] - indptr[b] == ceil(kv_len[b]/P).
 *     Kernels never read a page id outside [0, nnz), a pool row outside
 *     [0, num_blocks) nor a token at or past kv_len[b]: a request's page-id
 *     offsets are clamped to [0, nnz) and its range to the pages it has, and
 *     a page id outside [0, num_blocks) is read as pool row 0 on every
 *     kernel path. A malformed device CSR therefore gives wrong numbers for
 *     the requests it touches, never a fault. pdk_validate_csr checks a host
 *     copy.
 *   - Query: one token per request, q [batch, num_q_heads, head_dim_k] in f32
 *     or bf16, row major. Query head i reads KV head i / (Hq / Hkv)
 *     [cascade-PR, "The decomposition, and the one part that is not obvious"].
 */
#ifndef PDK_H
#define PDK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PDK_F32 = 0, PDK_BF16 = 1, PDK_FP8_E4M3 = 2 } pdk_dtype;

typedef enum {
  PDK_OK = 0,
  PDK_ERR_ARG = -1,          /* null pointer or out-of-range scalar */
  PDK_ERR_SHAPE = -2,        /* inconsistent sizes or page table */
  PDK_ERR_DTYPE = -3,        /* dtype not accepted by this entry point */
  PDK_ERR_UNSUPPORTED = -4,  /* valid, but no kernel instantiated for it */
  PDK_ERR_WORKSPACE = -5,    /* workspace too small or plan not uploaded */
  PDK_ERR_HIP = -6           /* a HIP runtime call failed */
} pdk_status;

/* Why a cascade plan fell back to the flat launch [cascade-PR, "Task items"
 * item 4, and "Proving which path a benchmark arm took"]. */
typedef enum {
  PDK_DECLINE_NONE = 0,
  PDK_DECLINE_DISABLED = 1,
  PDK_DECLINE_NO_CANDIDATE = 2,
  PDK_DECLINE_MEMBERS_BELOW_MIN = 3,
  PDK_DECLINE_SPAN_BELOW_MIN = 4,
  PDK_DECLINE_REACHES_LAST_PAGE = 5
} pdk_decline;

typedef struct {
  const void* k;          /* device, HND [num_blocks, Hkv, P, head_dim_k] */
  const void* v;          /* device, HND [num_blocks, Hkv, P, head_dim_v]; NULL: latent pool */
  int32_t num_blocks;
  int32_t page_size;      /* P, tokens per page */
  int32_t num_kv_heads;   /* Hkv */
  int32_t head_dim_k;
  int32_t head_dim_v;
  int32_t dtype;          /* pdk_dtype of k and v */
  float k_scale;          /* fp8 only: per-tensor dequant scale of k */
  float v_scale;          /* fp8 only: per-tensor dequant scale of v (latent: unused) */
} pdk_kv_pool;

typedef struct {
  const int32_t* indptr;  /* [batch + 1] */
  const int32_t* indices; /* [nnz] */
  const int32_t* kv_len;  /* [batch] */
  int32_t batch;
  int32_t nnz;            /* indptr[batch] */
} pdk_csr;

/* ---------------------------------------------------------------------- */
/* Host-side integer work                                                 */
/* ---------------------------------------------------------------------- */

/* Split-KV partitions [cascade-PR, "Test plan": cross-CTA split-KV with a
 * heuristic chunk size]: partitions tile each request's range from its first
 * token in partition_tokens steps, the last one short.
 * part_indptr[b+1] = part_indptr[b] + ceil(kv_len[b] / partition_tokens).
 * Host arrays: kv_len [batch] in, part_indptr [batch+1] out.
 * Errors: PDK_ERR_ARG (null, batch < 0, partition_tokens <= 0, kv_len < 0). */
int pdk_partition_indptr(const int32_t* kv_len, int32_t batch, int32_t partition_tokens,
                         int32_t* part_indptr);

/* Checks a host copy of a page table: indptr[0] == 0, monotone,
 * indptr[batch] == nnz, page counts == ceil(kv_len/P), ids in [0, num_blocks).
 * Returns PDK_OK or PDK_ERR_SHAPE with the first violation in pdk_last_error. */
int pdk_validate_csr(const pdk_csr* csr, int32_t page_size, int32_t num_blocks);

/* Kill-switch parse [cascade-PR, "Task items" item 4]: after trimming blanks
 * and ignoring case, 0/false/off/no -> 0 and 1/true/on/yes -> 1; anything
 * else, or NULL, -> -1 (the shipped default, which is off).
 * pdk_cascade_enabled_from_env reads the named environment variable. */
int pdk_parse_switch(const char* value);
int pdk_cascade_enabled_from_env(const char* var_name);

/* KV-head-major stacking [cascade-PR, "The decomposition"]: for every stacked
 * head h0 = kv*(M*G) + m*G + g, out[h0] = m*Hq + (kv*G + g), Hq = Hkv*G.
 * Host array out [M*Hq]. */
int pdk_stacked_head_map(int32_t num_members, int32_t num_kv_heads, int32_t group,
                         int32_t* out);

/* ---------------------------------------------------------------------- */
/* GPU kernels                                                            */
/* ---------------------------------------------------------------------- */

/* One normalized partial state per (request, partition, query head)
 * [cascade-PR, "The decomposition": one workgroup owns every query head of
 * one KV head for one (request, page tile) and loads each K/V element once].
 * csr_dev: device page table; part_indptr_dev: device [batch+1] from
 * pdk_partition_indptr; num_partitions = part_indptr[batch].
 * Outputs v_part [num_partitions, num_q_heads, head_dim_v] and
 * lse_part [num_partitions, num_q_heads], row = part_indptr[b] + p.
 * partition_tokens must be a positive multiple of page_size.
 * Dtypes: q f32|bf16; pool f32|bf16|fp8_e4m3 (fp8 is dequantized to bf16
 * with the pool's scale on load [DCP-PR, 3.2 figure, 3.3]).
 * Errors: PDK_ERR_ARG, PDK_ERR_SHAPE, PDK_ERR_DTYPE, PDK_ERR_UNSUPPORTED
 * (head dims / head counts without an instantiated kernel, or a partition of
 * more pages than the chosen kernel stages: partition_tokens / page_size at
 * most 1023 on the vector path and the head-dim-128 matrix-core path on
 * 1-2 token pages, 511 on the LDS-ring path (>= 16 rows per KV head, pages
 * of >= 4 tokens), 255 on the latent 576/512 paths), PDK_ERR_HIP. */
int pdk_paged_decode_partial(const pdk_kv_pool* pool, const pdk_csr* csr_dev, const void* q,
                             int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                             int32_t partition_tokens, const int32_t* part_indptr_dev,
                             int32_t num_partitions, float* v_part, float* lse_part,
                             hipStream_t stream);

/* Merge of states [cascade-PR, "How the #898 merge kernel is reused"]:
 * output row j combines input rows o_indptr[j] <= r < o_indptr[j+1]:
 * m = max lse_r, w_r = 2^(lse_r - m), l = sum w_r, v_out = sum w_r v_r / l,
 * lse_out = m + log2 l. Rows with lse = -inf are skipped; an empty group or
 * one with only -inf rows gives (0, -inf); a group of one row is copied
 * bit for bit (the identity the page relies on).
 * Device arrays: v_in [num_in, H, D], lse_in [num_in, H], o_indptr [num_out + 1],
 * v_out [num_out, H, D], lse_out [num_out, H] (may be NULL). Group bounds are
 * clamped to [0, num_in) on the device, so a bad o_indptr never reads past
 * the inputs. D must be a multiple of 4.
 * Errors: PDK_ERR_ARG, PDK_ERR_SHAPE, PDK_ERR_HIP. */
int pdk_merge_states(const float* v_in, const float* lse_in, int32_t num_in,
                     const int32_t* o_indptr_dev, int32_t num_out, int32_t num_heads,
                     int32_t head_dim, float* v_out, float* lse_out, hipStream_t stream);

/* Flat split-KV decode = pdk_paged_decode_partial + pdk_merge_states
 * [cascade-PR, "How the #898 merge kernel is reused": launch_with_lse returns
 * the (V, LSE) pair]. out [batch, Hq, head_dim_v], lse_out [batch, Hq]
 * (may be NULL). workspace: device, at least
 * pdk_decode_flat_workspace_bytes(num_partitions, Hq, head_dim_v) bytes. */
size_t pdk_decode_flat_workspace_bytes(int32_t num_partitions, int32_t num_q_heads,
                                       int32_t head_dim_v);
int pdk_decode_flat(const pdk_kv_pool* pool, const pdk_csr* csr_dev, const void* q,
                    int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                    int32_t partition_tokens, const int32_t* part_indptr_dev,
                    int32_t num_partitions, float* out, float* lse_out, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* pdk_decode_flat without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The partial states live in a static device array
 * of PDK_DECODE_FLAT_NOALLOC_MAX_BYTES (32 MiB), one per device, held from
 * the library's first use on that device until the process ends; its
 * address is looked up once per device on the first call there. Calls that
 * need more, pdk_decode_flat_workspace_bytes(num_partitions, Hq, head_dim_v)
 * > the maximum (at Hq 32 and head dim 128: more than 2,032 partitions),
 * fail with PDK_ERR_WORKSPACE before any launch. Nothing is allocated or
 * freed. Every call on one device shares that device's array: calls that
 * overlap on one device (two streams, or two host threads) race and give
 * wrong results; calls ordered on one stream are safe (each call writes
 * every state row it reads). Other arguments and errors: pdk_decode_flat. */
#define PDK_DECODE_FLAT_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int pdk_decode_flat_noalloc(const pdk_kv_pool* pool, const pdk_csr* csr_dev, const void* q,
                            int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                            int32_t partition_tokens, const int32_t* part_indptr_dev,
                            int32_t num_partitions, float* out, float* lse_out,
                            hipStream_t stream);

/* Multi-token steps: q_tokens = T >= 1 query tokens per request in one
 * step (verification of speculated tokens, chunked prefill of a few tokens).
 * q [batch, T, Hq, Dk] (f32|bf16); the request's range (kv_len tokens)
 * already holds the step's T new tokens as its last T tokens. causal = 1:
 * token t sees positions 0 .. kv_len[b] - T + t, its own and the earlier
 * ones; a token that sees nothing of a partition gets the empty state
 * (0, -inf) there. causal = 0: every token sees the whole range (a cached
 * prefix, [DCP-PR, 3.2 figure]: cached chunks are attended non-causally).
 * Outputs v_part [num_partitions, T, Hq, head_dim_v], lse_part
 * [num_partitions, T, Hq]. T = 1 gives pdk_paged_decode_partial's results
 * for either value of causal. Errors: as pdk_paged_decode_partial, plus
 * PDK_ERR_ARG for T < 1 or causal outside {0, 1}. */
int pdk_paged_multi_token_partial(const pdk_kv_pool* pool, const pdk_csr* csr_dev,
                                  const void* q, int32_t q_dtype, int32_t num_q_heads,
                                  int32_t q_tokens, int32_t causal, float sm_scale,
                                  int32_t partition_tokens, const int32_t* part_indptr_dev,
                                  int32_t num_partitions, float* v_part, float* lse_part,
                                  hipStream_t stream);

/* pdk_paged_multi_token_partial + pdk_merge_states over each request's
 * partitions, the (token, head) pairs merged as T*Hq heads. out
 * [batch, T, Hq, head_dim_v], lse_out [batch, T, Hq] (may be NULL).
 * workspace: device, at least
 * pdk_decode_flat_workspace_bytes(num_partitions, T * Hq, head_dim_v) bytes. */
int pdk_multi_token_flat(const pdk_kv_pool* pool, const pdk_csr* csr_dev, const void* q,
                         int32_t q_dtype, int32_t num_q_heads, int32_t q_tokens, int32_t causal,
                         float sm_scale, int32_t partition_tokens,
                         const int32_t* part_indptr_dev, int32_t num_partitions, float* out,
                         float* lse_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Stack the query heads of M members KV-head-major, [M, Hkv, G, D] ->
 * [Hkv, M, G, D] [cascade-PR, "The decomposition"]: q0[h0] = q[members[m],
 * kv*G + g] for h0 = kv*(M*G) + m*G + g. q [*, Hkv*G, D] (f32|bf16),
 * members_dev [M], q0 [M*Hkv*G, D] in q's dtype. */
int pdk_stack_heads(const void* q, int32_t q_dtype, const int32_t* members_dev,
                    int32_t num_members, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                    void* q0, hipStream_t stream);

/* The inverse on states: out[m, kv*G + g] = in0[kv*(M*G) + m*G + g] for
 * v [M*Hq, D] -> [M, Hq, D] and lse [M*Hq] -> [M, Hq] (lse pointers may both
 * be NULL). f32 device arrays. */
int pdk_unstack_heads(const float* v0, const float* lse0, int32_t num_members,
                      int32_t num_kv_heads, int32_t group, int32_t head_dim, float* v_out,
                      float* lse_out, hipStream_t stream);

/* fp8 E4M3FN -> bf16 with a per-tensor scale, exactly as the attention
 * kernels dequantize on load [DCP-PR, 3.2 figure]: bf16 = RNE_bf16(f32(x) *
 * scale) with the product rounded to nearest even in binary32 [OCP-FP8].
 * Device arrays in [n] (uint8), out [n] (bf16 bit patterns). */
int pdk_fp8_dequant_bf16(const uint8_t* in, int64_t n, float scale, uint16_t* out,
                         hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Cascade (shared-prefix) decode [cascade-PR, "Task items" items 1-4]     */
/* ---------------------------------------------------------------------- */

typedef struct {
  int32_t enabled;             /* -1: shipped default (off); 0: off; 1: on */
  int32_t min_shared_pages;    /* span threshold in pages (default 16), >= 1 */
  int32_t min_members;         /* member threshold (default 2), >= 2 */
  int32_t max_groups;          /* 1: the page's single subgroup (default);
                                  0: every qualifying group; k: the best k */
  int32_t l0_partition_tokens; /* level-0 partition size, multiple of P */
  int32_t l1_partition_tokens; /* level-1 (and flat) partition size, multiple of P */
  int32_t fuse_levels;         /* 1 (default): levels 0 and 1 in one grid when a
                                  fused kernel covers the shape (bf16 pool and
                                  queries, head dim 128, pages >= 16 tokens,
                                  3-4 query heads per KV head), bit-identical
                                  to two launches; 0: two launches */
  int32_t max_depth;           /* levels of shared spans: 1 (default) is the
                                  page's one shared level; k > 1 adds nested
                                  spans below a span (a tenant sub-prefix
                                  under a system prompt), up to k levels */
} pdk_cascade_params;

void pdk_cascade_params_default(pdk_cascade_params* params);

typedef struct pdk_cascade_plan pdk_cascade_plan;

/* Detect shared prefixes in a HOST page table and build the two-level plan
 * [cascade-PR, "Detection reads the page table, not the refcounts", "Task
 * items" 1, 2, 4]. Grouping by first page, positional longest common page
 * prefix capped to full pages, rejection of spans that reach a member's last
 * page or fall below the thresholds, selection by span*(members-1), ties to
 * the lowest first batch index. A declined plan is not an error: it returns
 * PDK_OK with a decline reason and runs the flat path. The plan is owned by
 * the library until pdk_cascade_plan_free. page_size must match the pool.
 * With max_depth > 1, nested spans follow below each selected span [the
 * page scopes a third level out in "What I left out"; merging is
 * associative, "How the #898 merge kernel is reused"]: the span's members
 * are grouped by their page at the span's end, and each subgroup passing the
 * same checks from that page on is a child span; spans are numbered level by
 * level (by first member within a level) and all of them form the level-0
 * view; a request's level-1 range starts after the deepest span holding it
 * and its merge group has one row per span holding it plus one. */
int pdk_cascade_plan_create(const pdk_csr* csr_host, int32_t page_size,
                            const pdk_cascade_params* params, pdk_cascade_plan** plan_out);
void pdk_cascade_plan_free(pdk_cascade_plan* plan);

/* Read-only views of the plan's host arrays (valid until the plan is freed). */
enum {
  PDK_PLAN_MEMBERS = 0,         /* [member slots] batch indices, level-0 order */
  PDK_PLAN_GROUP_INDPTR = 1,    /* [K+1] offsets of each span into MEMBERS */
  PDK_PLAN_SPAN_PAGES = 2,      /* [K] */
  PDK_PLAN_L0_INDPTR = 3,       /* [K+1] level-0 view */
  PDK_PLAN_L0_INDICES = 4,
  PDK_PLAN_L0_LEN = 5,          /* [K] tokens */
  PDK_PLAN_L1_INDPTR = 6,       /* [B+1] level-1 view (= flat view when declined) */
  PDK_PLAN_L1_INDICES = 7,
  PDK_PLAN_L1_LEN = 8,          /* [B] */
  PDK_PLAN_MERGE_INDPTR = 9,    /* [B+1] the page's pairing: 1 row per span holding
                                   the request, plus 1 */
  PDK_PLAN_FUSED_MERGE_INDPTR = 10, /* [B+1] rows per request in the single merge */
  PDK_PLAN_GROUP_OF = 11,       /* [B] outermost span of each request, -1 if none */
  PDK_PLAN_MEMBER_RANK = 12,    /* [B] rank within that span, -1 if none */
  PDK_PLAN_SPAN_START = 13,     /* [K] first page of each span (0 for outermost) */
  PDK_PLAN_SPAN_PARENT = 14,    /* [K] enclosing span, -1 for outermost */
  PDK_PLAN_NUM_FIELDS = 15
};
int pdk_cascade_plan_get(const pdk_cascade_plan* plan, int32_t field, const int32_t** data,
                         int32_t* len);

/* stats = {batch, members, shared_pages, shared_tokens, prefix_chunks,
 * suffix_chunks} [cascade-PR, "Proving which path a benchmark arm took"];
 * decline receives a pdk_decline. Either pointer may be NULL. */
int pdk_cascade_plan_stats(const pdk_cascade_plan* plan, int32_t stats[6], int32_t* decline);

/* Detection with the page ids on the device [cascade-PR, "Detection reads
 * the page table, not the refcounts"; "What I left out": detection re-runs
 * per layer per step]. csr_dev is the device page table (indptr, indices,
 * kv_len, batch, nnz); indptr_host / kv_len_host are host copies of its row
 * offsets [batch+1] and lengths [batch] (O(batch): what a scheduler keeps),
 * which must describe the device table (checked: offsets from 0 to at most nnz,
 * ceil(len / P) pages per request). A device kernel groups the requests by
 * first page and compares each with its group's first member; two ints per
 * request come back (the call synchronizes `stream`) and the host applies
 * the planner's rules, so the plan equals pdk_cascade_plan_create's for the
 * same table, except that the views' page ids are not copied to the host
 * (PDK_PLAN_L0_INDICES / PDK_PLAN_L1_INDICES read as empty): upload it with
 * pdk_cascade_plan_upload_device, which gathers them from csr_dev into the
 * workspace on `stream` (csr_dev must hold the same page ids then);
 * pdk_cascade_plan_upload refuses such a plan. scratch_dev: device memory
 * of pdk_cascade_device_detect_scratch_bytes(batch) bytes. Nested spans
 * (max_depth > 1) take one more detection per level of spans: each span's
 * members are compared from the span's end page on the device (the host
 * uploads a span key and that page offset per request, two ints per
 * request come back), and the host applies the child-span rules.
 * Errors: PDK_ERR_ARG, PDK_ERR_SHAPE, PDK_ERR_WORKSPACE, PDK_ERR_HIP. */
size_t pdk_cascade_device_detect_scratch_bytes(int32_t batch);
int pdk_cascade_plan_create_device(const pdk_csr* csr_dev, const int32_t* indptr_host,
                                   const int32_t* kv_len_host, int32_t page_size,
                                   const pdk_cascade_params* params, void* scratch_dev,
                                   size_t scratch_bytes, hipStream_t stream,
                                   pdk_cascade_plan** plan_out);
int pdk_cascade_plan_upload_device(pdk_cascade_plan* plan, const pdk_csr* csr_dev,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Plan memoization [cascade-PR, "What I left out, and where I was unsure":
 * detection re-runs per layer per step; a plan slot in the plan cache is the
 * follow-up]. A cache of up to `capacity` plans, least recently used out
 * first. The key is the whole HOST page table - indptr, indices AND kv_len -
 * with the page size and the parameters: a plan depends on the KV lengths,
 * not only on the rows [FreeToken issue "Layer-major prefill for offloaded
 * MoE": a plan cache keyed by rows was wrong once split-KV depended on KV
 * length]. pdk_plan_cache_get returns the cached plan for an equal key
 * (*hit = 1; content compared, not only hashed) or builds, caches and
 * returns a new one (*hit = 0). The plan is owned by the cache: do not free
 * it; it stays valid until a later get evicts it or the cache is freed, and
 * keeps its upload, so every layer of a step runs it from the same
 * workspace. *entry_id (may be NULL) is unique per built plan. Calls on one
 * cache are serialized by a mutex. Errors: as pdk_cascade_plan_create. */
typedef struct pdk_plan_cache pdk_plan_cache;
int pdk_plan_cache_create(int32_t capacity, pdk_plan_cache** cache_out);
void pdk_plan_cache_free(pdk_plan_cache* cache);
int pdk_plan_cache_get(pdk_plan_cache* cache, const pdk_csr* csr_host, int32_t page_size,
                       const pdk_cascade_params* params, pdk_cascade_plan** plan_out,
                       int64_t* entry_id, int32_t* hit);
/* stats = {lookups, hits, builds, evictions, entries} */
int pdk_plan_cache_stats(const pdk_plan_cache* cache, int64_t stats[5]);

/* Partition-size autotuning per shape bucket, cold cache [cascade-PR, "What
 * I left out, and where I was unsure": the shape-bucketed autotuner with
 * cold-L2 methodology is not wired to either cascade level, which use the
 * heuristic chunk size]. pdk_cascade_autotune builds the plan of every
 * candidate (level-0 size x level-1 size, each a positive multiple of
 * page_size), uploads it to `workspace` (at least
 * pdk_cascade_autotune_workspace_bytes) and times `reps` whole steps
 * (pdk_run_cascade_decode) on `stream` with HIP events, each after a read of
 * `flush_buffer` (device scratch of flush_bytes, e.g. 512 MiB, > the 256 MB
 * last-level cache; NULL: no flush), after two untimed steps. The fastest
 * pair is kept for the step's shape bucket (pdk_cascade_tuning_key: page
 * size, head counts and dims, dtypes, the plan's thresholds and switches,
 * and power-of-two buckets of batch, total tokens, shared tokens and
 * members); a later call in the same bucket returns it without measuring
 * (result->measured = 0). times_us (optional, [n_l0 * n_l1], l0-major) gets
 * each candidate's mean device us (-1 when nothing was measured). out /
 * lse_out receive the last candidate's outputs. Synchronizes `stream`.
 * pdk_cascade_tuned_params fills *tuned with the bucket's sizes (*found = 1)
 * or copies *params (*found = 0). The bucket table is process-wide and
 * guarded by a mutex; pdk_cascade_tuning_clear empties it. */
typedef struct {
  int32_t l0_partition_tokens;
  int32_t l1_partition_tokens;
  float us;         /* mean device microseconds per step of the chosen pair */
  int32_t measured; /* 1: measured by this call; 0: from the bucket table */
} pdk_tuning;
int pdk_cascade_tuning_key(const pdk_csr* csr_host, int32_t page_size,
                           const pdk_cascade_params* params, const pdk_kv_pool* pool,
                           int32_t num_q_heads, int32_t q_dtype, int32_t key[16]);
size_t pdk_cascade_autotune_workspace_bytes(const pdk_csr* csr_host, int32_t page_size,
                                            const pdk_cascade_params* params,
                                            const int32_t* l0_candidates, int32_t n_l0,
                                            const int32_t* l1_candidates, int32_t n_l1,
                                            int32_t num_q_heads, int32_t head_dim_v);
int pdk_cascade_autotune(const pdk_csr* csr_host, int32_t page_size,
                         const pdk_cascade_params* params, const pdk_kv_pool* pool, const void* q,
                         int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                         const int32_t* l0_candidates, int32_t n_l0,
                         const int32_t* l1_candidates, int32_t n_l1, int32_t reps,
                         void* flush_buffer, size_t flush_bytes, void* workspace,
                         size_t workspace_bytes, float* out, float* lse_out, float* times_us,
                         hipStream_t stream, pdk_tuning* result);
int pdk_cascade_tuned_params(const pdk_csr* csr_host, int32_t page_size,
                             const pdk_cascade_params* params, const pdk_kv_pool* pool,
                             int32_t num_q_heads, int32_t q_dtype, pdk_cascade_params* tuned,
                             int32_t* found);
void pdk_cascade_tuning_clear(void);

/* Device workspace for pdk_run_cascade_decode: the plan's integer arrays
 * followed by the partial states of both levels. */
size_t pdk_cascade_workspace_bytes(const pdk_cascade_plan* plan, int32_t num_q_heads,
                                   int32_t head_dim_v);

/* Copy the plan's integer arrays into the head of the workspace
 * (hipMemcpyAsync on stream). The plan must stay alive until the copy has
 * completed. Must precede pdk_run_cascade_decode with the same workspace. */
int pdk_cascade_plan_upload(pdk_cascade_plan* plan, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Run the plan [cascade-PR, "Task items" item 2]: one level-0 launch over
 * each selected group's span with the members' query heads stacked
 * KV-head-major (partials written straight into the members' rows), one
 * level-1 launch over every request's remaining range, then one merge per
 * request over [level-0 partitions][level-1 partitions] - equal to the
 * page's level merge followed by the pair merge, by associativity. A
 * declined plan runs the flat path. out [B, Hq, head_dim_v], lse_out [B, Hq]
 * (may be NULL). */
int pdk_run_cascade_decode(const pdk_cascade_plan* plan, const pdk_kv_pool* pool, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, float sm_scale, float* out,
                           float* lse_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* The two halves of pdk_run_cascade_decode, for callers that enqueue other
 * work (or timing events) between them: the level-0 and level-1 partial
 * launches into the workspace, then the single merge into out / lse_out.
 * Same arguments and errors; the merge needs the head dim of the values. */
int pdk_run_cascade_partials(const pdk_cascade_plan* plan, const pdk_kv_pool* pool,
                             const void* q, int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
int pdk_run_cascade_merge(const pdk_cascade_plan* plan, int32_t num_q_heads, int32_t head_dim_v,
                          float* out, float* lse_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Chunked cached prefix + new suffix (one GPU's share of MLA decode)      */
/* [DCP-PR, 3.2 figure]                                                    */
/* ---------------------------------------------------------------------- */

typedef struct pdk_chunked_plan pdk_chunked_plan;

/* Host-side split of each request's cached range into chunks of
 * chunk_tokens (aligned at token 0), each chunk into partitions of
 * partition_tokens; plus the suffix partitions. Both page tables are HOST
 * copies; chunk_tokens and partition sizes are multiples of their page sizes. */
int pdk_chunked_plan_create(const pdk_csr* prefix_host, int32_t prefix_page_size,
                            int32_t chunk_tokens, int32_t prefix_partition_tokens,
                            const pdk_csr* suffix_host, int32_t suffix_page_size,
                            int32_t suffix_partition_tokens, pdk_chunked_plan** plan_out);
void pdk_chunked_plan_free(pdk_chunked_plan* plan);
/* counts = {batch, chunks, prefix_partitions, suffix_partitions} */
int pdk_chunked_plan_counts(const pdk_chunked_plan* plan, int32_t counts[4]);
size_t pdk_chunked_workspace_bytes(const pdk_chunked_plan* plan, int32_t num_q_heads,
                                   int32_t head_dim_v);
int pdk_chunked_plan_upload(pdk_chunked_plan* plan, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* With chunk_out/chunk_lse (caller buffers [chunks, Hq, Dv] and
 * [chunks, Hq]): chunk partials -> merge per chunk (each chunk's (O, LSE),
 * written there) -> merge across each request's chunks -> suffix partials
 * and merge -> merge of the prefix state with the suffix state. With both
 * NULL: chunk and suffix partials, then ONE merge over all partials of each
 * request - the same merges regrouped (merging is associative, [cascade-PR,
 * "How the #898 merge kernel is reused"]), equal up to f32 rounding.
 * out [B, Hq, Dv], lse_out [B, Hq] (log2). */
int pdk_run_chunked_decode(const pdk_chunked_plan* plan, const pdk_kv_pool* prefix_pool,
                           const pdk_kv_pool* suffix_pool, const void* q, int32_t q_dtype,
                           int32_t num_q_heads, float sm_scale, float* out, float* lse_out,
                           float* chunk_out, float* chunk_lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* pdk_run_chunked_decode for a step of T = q_tokens query tokens per
 * request, q [B, T, Hq, Dk]: the cached chunks non-causally (every token
 * sees the whole cached prefix), the suffix causally (token t sees suffix
 * positions 0 .. suffix_len - T + t), then the same merges with the
 * (token, head) pairs as T*Hq heads. out [B, T, Hq, Dv], lse_out [B, T, Hq];
 * chunk_out/chunk_lse (optional) [chunks, T, Hq, Dv] / [chunks, T, Hq].
 * The workspace is pdk_chunked_workspace_bytes(plan, T * Hq, Dv) bytes,
 * uploaded with pdk_chunked_plan_upload. T = 1 is pdk_run_chunked_decode. */
int pdk_run_chunked_multi_token(const pdk_chunked_plan* plan, const pdk_kv_pool* prefix_pool,
                                const pdk_kv_pool* suffix_pool, const void* q, int32_t q_dtype,
                                int32_t num_q_heads, int32_t q_tokens, float sm_scale,
                                float* out, float* lse_out, float* chunk_out, float* chunk_lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step graphs: the kernel launches of one decode step recorded once by HIP
 * stream capture and replayed with one launch (a decode loop then makes one
 * host call per step). Between pdk_graph_begin(stream) and
 * pdk_graph_end(stream, &g) the caller makes run calls on `stream` only:
 * pdk_run_cascade_decode / _partials / _merge, pdk_run_chunked_decode /
 * _multi_token, pdk_decode_flat, pdk_paged_decode_partial, pdk_merge_states
 * (each only launches kernels). Plans must be uploaded, workspaces and
 * outputs allocated beforehand: nothing may allocate, copy from the host or
 * synchronize while recording, and stream must not be the null stream. A
 * replay (pdk_graph_launch, any stream) runs the recorded kernels with the
 * recorded arguments: it reads the current contents of every buffer the
 * calls named (queries, pools, device page tables, uploaded plans) and
 * writes the same outputs, so a plan may not be re-uploaded elsewhere or
 * freed while its graph lives. pdk_graph_end always ends the capture; on a
 * capture error it returns PDK_ERR_HIP and no graph. pdk_graph_nodes counts
 * the recorded kernel nodes and any other nodes (none for the calls above).
 * The graph is owned by the caller: pdk_graph_free. */
typedef struct pdk_graph pdk_graph;
int pdk_graph_begin(hipStream_t stream);
int pdk_graph_end(hipStream_t stream, pdk_graph** out);
int pdk_graph_launch(const pdk_graph* graph, hipStream_t stream);
int pdk_graph_nodes(const pdk_graph* graph, int32_t* kernel_nodes, int32_t* other_nodes);
void pdk_graph_free(pdk_graph* graph);

/* Thread-local description of the last non-OK status on this thread. */
const char* pdk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PDK_H */
