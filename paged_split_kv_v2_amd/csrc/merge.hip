// merge_states and the small permutation / conversion kernels (gfx950).
//
// merge_states [cascade-PR = mlxcel pull request "perf(core): compute shared
// prompt prefixes once per decode batch", section "How the #898 merge kernel
// is reused"]: v_in [N, H, D] rows each normalized by their own denominator,
// lse_in [N, H] in log2 units, o_indptr [M+1] grouping contiguous rows into
// output rows. A group of one row is the identity; the merge is associative.
//
// The merge is a pure stream (about 2 flops per loaded element), so it is
// laid out for HBM: each thread owns four consecutive floats of one output
// row (one 16-byte load per input row), a wave covers 256 floats of the
// [H, D] row, and a group's input rows are read sixteen at a time (their
// LSEs and 16-byte value loads issued together) and folded in with a running
// maximum, so a group of up to 16 rows costs one memory round trip. The
// waves of a workgroup take independent (output row, 256-float span) units.
// (Measured on 8192 output rows of 32 x 128 floats, 1-16 rows per group:
// sixteen rows per round trip 228 us against 243 us for eight, 219 us with
// non-temporal loads and stores, 208 us with the group bounds read through
// the scalar cache; issuing the loads from scalar row bases cuts
// registers to four waves per SIMD but runs slower, 235 us, and so does a
// grid-stride loop over units, 269 us.)

#include "device.h"
#include "internal.h"

namespace pdk {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Input rows are read once and output rows written once: non-temporal
// (streaming) loads and stores.
__device__ __forceinline__ float4 load_nt(const float* p) {
  const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

constexpr int kMergeThreads = 256;  // four independent waves per workgroup
constexpr int kMergeSpan = 64 * 4;  // floats of an output row per wave
constexpr int kMergeBatch = 16;     // input rows whose loads are issued together

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ v_in, const float* __restrict__ lse_in, int num_in,
    const int* __restrict__ o_indptr, int H, int D, int chunks, long long units,
    int out_stride, float* __restrict__ v_out, float* __restrict__ lse_out) {
  // the wave's unit, known wave-uniform: its group bounds come through the
  // scalar cache
  const long long unit = (long long)blockIdx.x * (kMergeThreads / 64) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (unit >= units) return;  // no barrier below
  const int i = (int)(unit / chunks);
  const int c = (int)(unit - (long long)i * chunks);
  const int HD = H * D;
  const int e = c * kMergeSpan + (threadIdx.x & 63) * 4;
  if (e >= HD) return;  // no barrier below
  const int head = e / D;
  // group bounds clamped to the input rows
  const int a = min(max(o_indptr[i], 0), num_in);
  const int n = min(max(o_indptr[i + 1], a), num_in) - a;
  const size_t orow = (size_t)i * out_stride * HD + e;

  float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = -INFINITY;
  const float* lrow = lse_in + (size_t)a * H + head;
  const float lse0 = n > 0 ? lrow[0] : -INFINITY;
  if (n == 1 && lse0 != -INFINITY) {
    // identity, bit for bit
    out = load_nt(v_in + (size_t)a * HD + e);
    lse = lse0;
  } else if (n > 1) {
    // one pass in batches of kMergeBatch rows: the batch's LSEs and value
    // rows are loaded together, then folded in with a running maximum (for
    // groups of at most kMergeBatch rows this is the plain two-step merge)
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* vrow = v_in + (size_t)a * HD + e;
    for (int r0 = 0; r0 < n; r0 += kMergeBatch) {
      float w[kMergeBatch];
      float4 x[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const bool in = r0 + k < n;
        w[k] = in ? lrow[(size_t)(r0 + k) * H] : -INFINITY;
        x[k] = in ? load_nt(vrow + (size_t)(r0 + k) * HD) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float bm = w[0];
#pragma unroll
      for (int k = 1; k < kMergeBatch; ++k) bm = fmaxf(bm, w[k]);
      if (bm == -INFINITY) continue;  // only empty states in this batch
      if (bm > m) {
        const float c = (m == -INFINITY) ? 0.f : fast_exp2(m - bm);
        l *= c;
        acc = make_float4(acc.x * c, acc.y * c, acc.z * c, acc.w * c);
        m = bm;
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        if (w[k] == -INFINITY) continue;  // empty state: not read into the sum
        const float wk = fast_exp2(w[k] - m);
        l += wk;
        acc.x = fmaf(wk, x[k].x, acc.x);
        acc.y = fmaf(wk, x[k].y, acc.y);
        acc.z = fmaf(wk, x[k].z, acc.z);
        acc.w = fmaf(wk, x[k].w, acc.w);
      }
    }
    if (m != -INFINITY) {
      out = make_float4(acc.x / l, acc.y / l, acc.z / l, acc.w / l);
      lse = m + log2f(l);
    }
  }
  __builtin_nontemporal_store(f32x4_t{out.x, out.y, out.z, out.w},
                              reinterpret_cast<f32x4_t*>(v_out + orow));
  if (lse_out != nullptr && (e - head * D) == 0) lse_out[(size_t)i * out_stride * H + head] = lse;
}

// q0[kv*(M*G) + m*G + g, :] = q[members[m], kv*G + g, :]
template <typename T>
__global__ void stack_kernel(const T* __restrict__ q, const int* __restrict__ members, int M,
                             int Hkv, int G, int D, T* __restrict__ q0) {
  const long long total = (long long)M * Hkv * G * D;
  for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < total;
       x += (long long)gridDim.x * blockDim.x) {
    const int d = (int)(x % D);
    const long long h0 = x / D;
    const int g = (int)(h0 % G);
    const int m = (int)((h0 / G) % M);
    const int kv = (int)(h0 / ((long long)G * M));
    const int Hq = Hkv * G;
    q0[x] = q[((size_t)members[m] * Hq + kv * G + g) * D + d];
  }
}

// out[m, kv*G + g, :] = v0[kv*(M*G) + m*G + g, :] (and the same for lse)
__global__ void unstack_kernel(const float* __restrict__ v0, const float* __restrict__ lse0,
                               int M, int Hkv, int G, int D, float* __restrict__ v_out,
                               float* __restrict__ lse_out) {
  const long long total = (long long)M * Hkv * G * D;
  for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < total;
       x += (long long)gridDim.x * blockDim.x) {
    const int d = (int)(x % D);
    const long long h0 = x / D;
    const int g = (int)(h0 % G);
    const int m = (int)((h0 / G) % M);
    const int kv = (int)(h0 / ((long long)G * M));
    const size_t o = (size_t)m * Hkv * G + kv * G + g;
    v_out[o * D + d] = v0[x];
    if (d == 0 && lse0 != nullptr) lse_out[o] = lse0[h0];
  }
}

__global__ void dequant_kernel(const uint8_t* __restrict__ in, long long n, float scale,
                               uint16_t* __restrict__ out) {
  for (long long x = (blockIdx.x * (long long)blockDim.x + threadIdx.x) * 4; x < n;
       x += (long long)gridDim.x * blockDim.x * 4) {
    uint32_t w = 0;
    const int k = (int)min(4LL, n - x);
    for (int i = 0; i < k; ++i) w |= (uint32_t)in[x + i] << (8 * i);
    uint32_t p01, p23;
    fp8x4_dequant_bf16(w, scale, p01, p23);
    const uint32_t bits[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
    for (int i = 0; i < k; ++i) out[x + i] = (uint16_t)bits[i];
  }
}

int check_launch(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PDK_ERR_HIP, "%s launch: %s", what, hipGetErrorString(err));
  return PDK_OK;
}

unsigned grid_for(long long items, int threads) {
  long long g = (items + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;  // grid-stride loops cover the rest
  return (unsigned)g;
}

}  // namespace

int launch_merge(const float* v_in, const float* lse_in, int num_in, const int* o_indptr,
                 int num_out, int H, int D, float* v_out, float* lse_out, int out_stride,
                 hipStream_t stream) {
  if (num_out == 0) return PDK_OK;
  const int chunks = (H * D + kMergeSpan - 1) / kMergeSpan;
  const long long units = (long long)num_out * chunks;
  const long long blocks = (units + kMergeThreads / 64 - 1) / (kMergeThreads / 64);
  if (blocks > 0x7FFFFFFFLL) return fail(PDK_ERR_SHAPE, "merge grid too large");
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, v_in,
                     lse_in, num_in, o_indptr, H, D, chunks, units, out_stride, v_out, lse_out);
  return check_launch("merge_states");
}

int launch_stack(const void* q, int q_dtype, const int* members, int M, int Hkv, int G, int D,
                 void* q0, hipStream_t stream) {
  const long long total = (long long)M * Hkv * G * D;
  if (total == 0) return PDK_OK;
  if (q_dtype == PDK_F32)
    hipLaunchKernelGGL(stack_kernel<float>, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                       (const float*)q, members, M, Hkv, G, D, (float*)q0);
  else
    hipLaunchKernelGGL(stack_kernel<uint16_t>, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                       (const uint16_t*)q, members, M, Hkv, G, D, (uint16_t*)q0);
  return check_launch("stack_heads");
}

int launch_unstack(const float* v0, const float* lse0, int M, int Hkv, int G, int D,
                   float* v_out, float* lse_out, hipStream_t stream) {
  const long long total = (long long)M * Hkv * G * D;
  if (total == 0) return PDK_OK;
  hipLaunchKernelGGL(unstack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, v0, lse0,
                     M, Hkv, G, D, v_out, lse_out);
  return check_launch("unstack_heads");
}

int launch_dequant(const uint8_t* in, long long n, float scale, uint16_t* out,
                   hipStream_t stream) {
  if (n == 0) return PDK_OK;
  hipLaunchKernelGGL(dequant_kernel, dim3(grid_for((n + 3) / 4, 256)), dim3(256), 0, stream, in,
                     n, scale, out);
  return check_launch("fp8 dequant");
}

}  // namespace pdk
