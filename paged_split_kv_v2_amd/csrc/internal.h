// Internal declarations shared by the host library and the HIP kernels.
// Not part of the public ABI (see include/pdk.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


#include "pdk.h"

namespace pdk {

// Arguments of one partial-state launch over a page-table "view".
//
// A view is a CSR page table plus partitions over it. In a flat (or
// level-1) launch, request b of the view is batch request b and owns
// G = Hq/Hkv query rows per KV head. In a stacked (level-0) launch, view
// request k is a group of members; it owns M_k * G query rows per KV head,
// row j = m*G + g taking member m's query head kv*G + g (KV-head-major
// stacking), and each member's partials go to that member's own output rows.
struct PartialArgs {
  // pool
  const void* k;
  const void* v;              // nullptr: latent pool, V = first Dv lanes of K
  long long k_bstride;        // elements between pool rows (blocks)
  long long k_hstride;        // elements between KV heads of a row
  long long v_bstride, v_hstride;
  int num_blocks, P, Hkv, Dk, Dv;
  int p_shift;                // log2(P) when P is a power of two, else -1
  int kv_dtype;
  float k_scale, v_scale;
  // view
  const int* indptr;
  const int* indices;
  const int* kv_len;
  int batch;
  int nnz;                    // page ids in indices; every read is clamped to [0, nnz)
  const int* part_indptr;     // [batch+1] partitions of the view
  int num_parts;
  int S;                      // partition tokens
  // queries
  const void* q;              // [*, Hq, Dk]
  int q_dtype;
  int Hq;
  int G;                      // query heads per KV head of the batch layout
  float scale_log2;           // sm_scale * log2(e)
  // multi-token steps (flat views only): q is [B, T, Hq, Dk], states are
  // [rows, T, Hq, Dv]; causal: token t sees positions <= kv_len - T + t
  int q_tokens;               // T >= 1
  int causal;
  // stacking; member_indptr == nullptr for a flat view
  const int* member_indptr;   // [batch+1] members of view request k
  const int* members;         // batch index of each member slot
  int max_rows;               // max query rows per KV head over the view
  // outputs [rows, Hq, Dv] and [rows, Hq]
  const int* out_row_base;    // flat: indexed by b; stacked: by member slot
  float* v_out;
  float* lse_out;
  // planned launches: workgroup item i is (view request, partition) work[i]
  const int2* work;           // nullptr: partition rows in part_indptr order
};

int launch_partial(const PartialArgs& a, hipStream_t stream);
int launch_partial_valu(const PartialArgs& a, hipStream_t stream);
// Launches on the matrix cores when an instantiation covers the shape
// (bf16 queries, >= 16 query rows per KV head); *handled says whether it did.
int launch_partial_mfma(const PartialArgs& a, hipStream_t stream, bool* handled);
// Latent (MLA) pools, 576/512 head dims, bf16 queries, >= 64 query rows.
int launch_partial_latent(const PartialArgs& a, hipStream_t stream, bool* handled);
// bf16 K/V pools of head dim 128 with bf16 queries, K/V staged by
// global->LDS loads, products on the matrix cores.
int launch_partial_dma(const PartialArgs& a, hipStream_t stream, bool* handled);
int valu_max_rows(int head_dim);
// Level 0 (a0, stacked) and level 1 (a1, flat) of a cascade step in one
// grid, when both fit the fused kernel's instantiations (*handled); the
// partial rows equal those of two launch_partial calls.
int launch_cascade_partials(const PartialArgs& a0, const PartialArgs& a1, hipStream_t stream,
                            bool* handled);
// out_stride: output row i is written at row i * out_stride of v_out / lse_out
int launch_merge(const float* v_in, const float* lse_in, int num_in, const int* o_indptr,
                 int num_out, int H, int D, float* v_out, float* lse_out, int out_stride,
                 hipStream_t stream);

// Checked entry points used by the plan runners (same checks as the public
// pdk_paged_decode_partial / pdk_merge_states, plus stacking and row maps).
// work: optional longest-first (view request, partition) items, one per
// partition of the view, that replace the part_indptr order.
// q_tokens / causal: multi-token steps (q [*, T, Hq, Dk], states
// [*, T, Hq, Dv]); causal masking only on flat views.
int partial_rows(const pdk_kv_pool* pool, const pdk_csr* view, const void* q, int q_dtype, int Hq,
                 float sm_scale, int S, const int* part_indptr, int num_parts,
                 const int* member_indptr, const int* members, int max_members, int G,
                 const int* out_row_base, float* v_out, float* lse_out, hipStream_t stream,
                 const int2* work = nullptr, int q_tokens = 1, int causal = 0);
// The checks of partial_rows, filling *out instead of launching; *empty
// when the view has nothing to compute.
int partial_args(const pdk_kv_pool* pool, const pdk_csr* view, const void* q, int q_dtype, int Hq,
                 float sm_scale, int S, const int* part_indptr, int num_parts,
                 const int* member_indptr, const int* members, int max_members, int G,
                 const int* out_row_base, float* v_out, float* lse_out, const int2* work,
                 PartialArgs* out, bool* empty, int q_tokens = 1, int causal = 0);
int merge_rows(const float* v_in, const float* lse_in, int num_in, const int* o_indptr,
               int num_out, int H, int D, float* v_out, float* lse_out, int out_stride,
               hipStream_t stream);
int launch_stack(const void* q, int q_dtype, const int* members, int M, int Hkv, int G, int D,
                 void* q0, hipStream_t stream);
int launch_unstack(const float* v0, const float* lse0, int M, int Hkv, int G, int D,
                   float* v_out, float* lse_out, hipStream_t stream);
int launch_dequant(const uint8_t* in, long long n, float scale, uint16_t* out,
                   hipStream_t stream);
// Device detection of shared pages: leader[b] (first request with the same
// page at position off[b] among those with key[b], -1 for a request without
// that page) and common[b] (page ids from off[b] shared with the leader).
// key and off (device [B], both or neither): without them, the first page
// of every request. The row offsets must describe [0, nnz).
int launch_detect(const int32_t* indptr, const int32_t* indices, const int32_t* kv_len,
                  const int32_t* key, const int32_t* off, int B, int32_t* leader,
                  int32_t* common, hipStream_t stream);
// dst[segs[3i+1] + j] = src[segs[3i] + j] for j < segs[3i+2] (device arrays).
int launch_gather_pages(const int32_t* src, const int32_t* segs, int nseg, int32_t* dst,
                        hipStream_t stream);

// error reporting (thread-local message, see pdk_last_error)
int fail(int status, const char* fmt, ...);


}  // namespace pdk
