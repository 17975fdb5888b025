// Device helpers for gfx950 (CDNA4, wave64): number formats and
// cross-lane reductions. Included by the .hip translation units only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 is the high half of a binary32: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return bits_f32(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return bits_f32(pair & 0xFFFF0000u); }

// binary32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// Two at once (one v_cvt_pk_bf16_f32), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Four OCP E4M3FN codes (one per byte of `w`) -> binary32, exact
// (v_cvt_pk_f32_fp8: gfx950 implements the OCP encoding).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float out[4]) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

// fp8 -> bf16 dequant with a per-tensor scale: RNE_bf16(RNE_f32(x * scale)).
// Returns two packed bf16 pairs for the four codes in `w`.
__device__ __forceinline__ void fp8x4_dequant_bf16(uint32_t w, float scale, uint32_t& p01,
                                                   uint32_t& p23) {
  float f[4];
  fp8x4_to_f32(w, f);
  p01 = pack_bf16x2_rne(f[0] * scale, f[1] * scale);
  p23 = pack_bf16x2_rne(f[2] * scale, f[3] * scale);
}

// DPP lane moves inside a row of 16 lanes. Every source lane exists for the
// patterns below, so bound_ctrl is set and no "old" value is needed (the move
// folds into the consuming VALU op as a DPP operand).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
enum : int {
  DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
};

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<DPP_QUAD_XOR1>(x);
  x += dpp_f32<DPP_QUAD_XOR2>(x);
  x += dpp_f32<DPP_ROW_HALF_MIRROR>(x);
  x += dpp_f32<DPP_ROW_MIRROR>(x);
  return x;
}

// The same all-reduce over N independent values, one stage at a time, so
// that consecutive DPP reads never wait on the VALU write before them.
template <int N>
__device__ __forceinline__ void row16_sum_n(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<DPP_QUAD_XOR1>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<DPP_QUAD_XOR2>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<DPP_ROW_HALF_MIRROR>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_f32<DPP_ROW_MIRROR>(x[i]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pdk
