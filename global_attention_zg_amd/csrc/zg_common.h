// Internal helpers shared by the gfx950 kernels of libzgattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head dim (the only one supported)
constexpr int kMaxRopeHalf = 32; // rope_dim <= head_dim / 2
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Revolutions per position of each rotary pair t: theta^(-2t/R) / (2*pi),
// computed in double on the host.  Angles are formed in double and reduced
// to [-1/2, 1/2] revolution before the float sine/cosine, so that positions
// up to 2^31 keep ~1e-7 rad accuracy.
struct RopeTable {
  double rev[kMaxRopeHalf];
};

__device__ __forceinline__ void rope_cos_sin(const RopeTable& tab, int t, long long pos,
                                             float& c, float& s) {
  double r = (double)pos * tab.rev[t];
  r -= rint(r);
  float f = (float)r;
  // v_sin_f32 / v_cos_f32 take their argument in revolutions.
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void unpack_bf16x8(u32x4 u, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(u[i]);
    x[2 * i + 1] = bf_hi(u[i]);
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Value held by lane (l ^ 32) combined with ours by a symmetric op: after
// v_permlane32_swap of (x, x), r[0] and r[1] hold the two halves' values of
// the pair {l, l^32} in some order.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sigmoid(g) = 1 / (1 + e^-g): exactly 1 for g = +inf and 0 for g = -inf.
__device__ __forceinline__ float sigmoidf_(float g) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-g * kLog2e));
}

}  // namespace zg
