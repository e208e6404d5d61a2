// E4M3 (OCP FP8: sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
// finite 448, no infinities) conversions used by the FP8 kernels.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 前置知识 ›
// FP8 混合精度训练与 TWEO: forward matrix multiplies in E4M3 with per-tensor
// scaling factors.  A tensor x with scale s is stored as the codes of
// x * s rounded to the nearest E4M3 value (ties to even) after clamping to
// [-448, 448]; its stored value is decode(code) / s.
#pragma once

#include "zg_common.h"

namespace zg {

constexpr float kE4M3Max = 448.0f;

// 32 bytes per lane: an A or B operand of the FP8 MFMAs (v_mfma_scale_*_f8f6f4)
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Codes of x[0..7] * scale (product in fp32, clamped, then v_cvt_pk_fp8_f32,
// which rounds to nearest even), bytes in element order.
__device__ __forceinline__ uint2 pack_e4m3x8(const float* x, float scale) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(x[e] * scale, -kE4M3Max), kE4M3Max);
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Four E4M3 codes (bytes of w) -> four bf16 values, exactly: every E4M3
// value is a bf16 value (3 mantissa bits <= 7, exponents 2^-9..2^8).
__device__ __forceinline__ void widen_e4m3x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Eight E4M3 codes -> eight bf16 values in element order.
__device__ __forceinline__ u32x4 widen_e4m3x8(uint2 c) {
  uint32_t a, b, d, e;
  widen_e4m3x4(c.x, a, b);
  widen_e4m3x4(c.y, d, e);
  return u32x4{a, b, d, e};
}

__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

}  // namespace zg
