// Shared-prefix detection on the device, for page tables that live on the
// GPU [cascade-PR, "Detection reads the page table, not the refcounts":
// equal page ids at equal positions are shared bytes; candidates group by
// their first page and share their longest common page prefix]. The two
// O(nnz) parts run here - grouping by first page and the positional
// comparison with the group's first member - and the host reads back two
// ints per request; every rule past that (caps, thresholds, scores,
// selection) is the host planner's. A second kernel gathers the views' page
// ids into the workspace when the plan is uploaded.

#include "device.h"
#include "internal.h"

namespace pdk {

namespace {

// One wave per request b, comparing page ids from position o = off[b]
// (0 without offsets) among the requests of b's span key[b] (all requests
// without keys): its leader is the smallest b' <= b with the same key and
// offset whose page at o is b's (64 candidates per ballot), and common[b]
// the number of page ids from o that b shares with it position by position
// (64 per ballot). Requests with a negative offset, no page at o or no
// token get leader -1. Without keys and offsets this is the grouping by
// first page of the two-level plan; with them, the grouping of a span's
// members by their page at the span's end that nested spans need.
__global__ __launch_bounds__(64) void detect_kernel(const int32_t* __restrict__ indptr,
                                                    const int32_t* __restrict__ indices,
                                                    const int32_t* __restrict__ kv_len,
                                                    const int32_t* __restrict__ key,
                                                    const int32_t* __restrict__ off, int B,
                                                    int32_t* __restrict__ leader,
                                                    int32_t* __restrict__ common) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int p0 = indptr[b];
  const int np = indptr[b + 1] - p0;
  const int o = off ? off[b] : 0;
  const int k = key ? key[b] : 0;
  if (o < 0 || np <= o || kv_len[b] < 1) {
    if (lane == 0) {
      leader[b] = -1;
      common[b] = 0;
    }
    return;
  }
  const int first = indices[p0 + o];
  int L = b;
  for (int base = 0; base < b; base += 64) {
    const int c = base + lane;
    bool hit = false;
    if (c < b && (!key || (key[c] == k && off[c] == o))) {
      const int q0 = indptr[c];
      hit = indptr[c + 1] - q0 > o && kv_len[c] >= 1 && indices[q0 + o] == first;
    }
    const unsigned long long m = __ballot(hit);
    if (m) {
      L = base + __ffsll((long long)m) - 1;
      break;
    }
  }
  int shared = np - o;
  if (L != b) {
    const int l0 = indptr[L] + o;
    const int n = min(np, indptr[L + 1] - indptr[L]) - o;
    shared = n;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const bool diff = i < n && indices[p0 + o + i] != indices[l0 + i];
      const unsigned long long m = __ballot(diff);
      if (m) {
        shared = base + __ffsll((long long)m) - 1;
        break;
      }
    }
  }
  if (lane == 0) {
    leader[b] = L;
    common[b] = shared;
  }
}

// One workgroup per segment (source offset, destination offset, count).
__global__ __launch_bounds__(256) void gather_pages_kernel(const int32_t* __restrict__ src,
                                                           const int32_t* __restrict__ segs,
                                                           int32_t* __restrict__ dst) {
  const int s = segs[3 * blockIdx.x], d = segs[3 * blockIdx.x + 1], n = segs[3 * blockIdx.x + 2];
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[d + i] = src[s + i];
}

}  // namespace

int launch_detect(const int32_t* indptr, const int32_t* indices, const int32_t* kv_len,
                  const int32_t* key, const int32_t* off, int B, int32_t* leader,
                  int32_t* common, hipStream_t stream) {
  if (B <= 0) return PDK_OK;
  if ((key == nullptr) != (off == nullptr))
    return fail(PDK_ERR_ARG, "detection keys and offsets go together");
  hipLaunchKernelGGL(detect_kernel, dim3(B), dim3(64), 0, stream, indptr, indices, kv_len, key,
                     off, B, leader, common);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "detect launch: %s", hipGetErrorString(e));
  return PDK_OK;
}

int launch_gather_pages(const int32_t* src, const int32_t* segs, int nseg, int32_t* dst,
                        hipStream_t stream) {
  if (nseg <= 0) return PDK_OK;
  hipLaunchKernelGGL(gather_pages_kernel, dim3(nseg), dim3(256), 0, stream, src, segs, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
  return PDK_OK;
}

}  // namespace pdk
