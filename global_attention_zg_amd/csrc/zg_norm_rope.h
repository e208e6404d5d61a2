// QK-RMSNorm + partial RoPE of one 128-value row spread over 16 lanes,
// shared by the key prologue and the decode kernels so that a key gets the
// same bits whichever kernel writes it to the cache.
//
// Page "7B 打 235B？中关村学院把'小模型怎么活'这道题答成了一份全开源配方"
// (shibing624.github.io), section 🏗️ 架构: Q and K are normalised with
// RMSNorm and rotated with RoPE on a 0.33 fraction of the head dim.
#pragma once

#include "zg_common.h"

namespace zg {

// The per-lane constants of the row code: the lane's 8 norm weights and the
// frequencies of its rotary angles t = c16 and c16 + 16 (rope_half <= 32).
// Kernels that loop over rows load them once, so that no global load sits
// between a prefetch and its use inside the loop.
struct RowConsts {
  float wl[8];
  uint64_t fr0, fr1;
};
static_assert(kMaxRopeHalf <= 32, "two rotary angles per lane");

__device__ __forceinline__ RowConsts row_consts(const float* w, int rope_half, const RopeTable& tab,
                                                int c16) {
  RowConsts k;
  const u32x4 w0 = ld16(w + 8 * c16);
  const u32x4 w1 = ld16(w + 8 * c16 + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k.wl[i] = __uint_as_float(w0[i]);
    k.wl[4 + i] = __uint_as_float(w1[i]);
  }
  k.fr0 = c16 < rope_half ? tab.frac[c16] : 0;
  k.fr1 = c16 + 16 < rope_half ? tab.frac[c16 + 16] : 0;
  return k;
}

// Normalise + rotate one row held as 8 values per lane (lane c16 = 0..15 of
// the row owns dims 8*c16 .. 8*c16+7).  `xs` is the row's LDS scratch.  The
// rotary cosines / sines live in per-row LDS tables; rows at the same
// position (the heads of one token) share them: the block's first row of
// each position (`own` true) fills its table, one angle per lane t % 16, and
// every row reads the table `cs_r` / `sn_r` of that first row.  Every thread
// of the block calls this together (one barrier, which waits for LDS only:
// global loads in flight stay in flight).
__device__ __forceinline__ void norm_rope_row(float* x, int c16, const RowConsts& k, float eps,
                                              int rope_half, long long pos, float* xs, bool own,
                                              float* cs_w, float* sn_w, const float* cs_r,
                                              const float* sn_r) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  // reduce over the 16 lanes of this row
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 16);
  const float r = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= r * k.wl[i];
  if (rope_half == 0) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) xs[8 * c16 + i] = x[i];
  if (own) {
    if (c16 < rope_half) rope_cos_sin_f(k.fr0, pos, cs_w[c16], sn_w[c16]);
    if (c16 + 16 < rope_half) rope_cos_sin_f(k.fr1, pos, cs_w[c16 + 16], sn_w[c16 + 16]);
  }
  lds_barrier();
  const int R = 2 * rope_half;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = 8 * c16 + i;
    if (d < R) {
      const int t = d < rope_half ? d : d - rope_half;
      const float c = cs_r[t], s = sn_r[t];
      if (d < rope_half)
        x[i] = x[i] * c - xs[d + rope_half] * s;
      else
        x[i] = x[i] * c + xs[d - rope_half] * s;
    }
  }
}

// The same for a single row (decode): loads the lane constants itself.
__device__ __forceinline__ void norm_rope_row(float* x, int c16, const float* w, float eps,
                                              int rope_half, const RopeTable& tab,
                                              long long pos, float* xs, bool own, float* cs_w,
                                              float* sn_w, const float* cs_r, const float* sn_r) {
  norm_rope_row(x, c16, row_consts(w, rope_half, tab, c16), eps, rope_half, pos, xs, own, cs_w,
                sn_w, cs_r, sn_r);
}

}  // namespace zg
