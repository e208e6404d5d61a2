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

// Revolutions per position of each rotary pair t, theta^(-2t/R) / (2*pi), as
// a 0.64 fixed-point fraction (computed on the host in extended precision).
// The angle of position p is then frac(p * rev) = (p * F mod 2^64) / 2^64,
// exact modular integer arithmetic for any 64-bit p; its top 32 bits, read
// as a signed number, give the angle reduced to [-1/2, 1/2) revolution with
// an error below 2^-32 revolution.
struct RopeTable {
  uint64_t frac[kMaxRopeHalf];
};

__device__ __forceinline__ void rope_cos_sin_f(uint64_t f, long long pos, float& c, float& s) {
  const uint64_t p = (uint64_t)pos;
  const uint32_t pl = (uint32_t)p, ph = (uint32_t)(p >> 32);
  const uint32_t fl = (uint32_t)f, fh = (uint32_t)(f >> 32);
  // bits 32..63 of p * f (the carry out of bits 0..31 is dropped: < 2^-32)
  const uint32_t top = __umulhi(pl, fl) + pl * fh + ph * fl;
  const float r = (float)(int32_t)top * 2.3283064365386963e-10f;  // * 2^-32
  // v_sin_f32 / v_cos_f32 take their argument in revolutions.
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

__device__ __forceinline__ void rope_cos_sin(const RopeTable& tab, int t, long long pos,
                                             float& c, float& s) {
  rope_cos_sin_f(tab.frac[t], pos, c, s);
}

// Workgroup barrier that waits for this wave's LDS operations only (the
// release fence of __syncthreads() also waits for every global load in
// flight, which would end any prefetch across the barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
