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

// Normalise + rotate one row held as 8 values per lane (lane c16 = 0..15 of
// the row owns dims 8*c16 .. 8*c16+7).  `xs` is the row's LDS scratch.  The
// rotary cosines / sines live in per-row LDS tables; rows at the same
// position (the heads of one token) share them: the block's first row of
// each position (`own` true) fills its table, one angle per lane t % 16, and
// every row reads the table `cs_r` / `sn_r` of that first row.  Every thread
// of the block calls this together (one barrier).
__device__ __forceinline__ void norm_rope_row(float* x, int c16, const float* w, float eps,
                                              int rope_half, const RopeTable& tab,
                                              long long pos, float* xs, bool own, float* cs_w,
                                              float* sn_w, const float* cs_r, const float* sn_r) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  // reduce over the 16 lanes of this row
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 16);
  const float r = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  const u32x4 w0 = ld16(w + 8 * c16);
  const u32x4 w1 = ld16(w + 8 * c16 + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] *= r * __uint_as_float(w0[i]);
    x[4 + i] *= r * __uint_as_float(w1[i]);
  }
  if (rope_half == 0) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) xs[8 * c16 + i] = x[i];
  if (own)
    for (int t = c16; t < rope_half; t += 16) rope_cos_sin(tab, t, pos, cs_w[t], sn_w[t]);
  __syncthreads();
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

}  // namespace zg
