// Tile-level building blocks of the gfx950 flash-attention forward kernels
// of libzgattn: the S^T = K' Q'^T and O^T += V^T P^T products on
// v_mfma_f32_32x32x16_bf16 with their LDS operand reads, the causal/band
// mask, the online softmax with lazy rescaling, and the fused query
// prologue (RMSNorm + partial RoPE) that turns raw query rows into the
// B operand of the score products.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 核心方法 (QK-RMSNorm, partial RoPE over a third of the head dims)
// and section 前置知识 › 滑动窗口注意力(SWA)与混合注意力 (the causal band).
#pragma once

#include "zg_common.h"
#include "zg_launch.h"
#include "zg_lds.h"

namespace zg {
namespace flash {

constexpr int kBN = 32;                          // keys per KV tile (one MFMA block)
constexpr int kRowBytes = kD * 2;                // 256-byte K'/V rows in LDS, 16-byte chunks XOR-swizzled
constexpr int kTileBytes = kBN * kRowBytes;      // 8192 per K' or V stage
constexpr float kRescaleThreshold = 8.0f;        // exp2 units

struct Geo {
  int heads_per_wg;  // query heads per workgroup (= waves sharing positions)
  int pos_per_wg;    // query positions per workgroup
  int n_pos_blocks;
  int hgroups;       // workgroups per (b, kv head, position block)
  int n_bhg;         // B * Hkv * hgroups
  // persistent causal grid: jobs (= position blocks x n_bhg) and work queues
  int n_jobs;
  int nq;
};

struct TileState {
  f32x16 acc[4];
  float m_run;   // running max of raw scores (this lane's query row)
  float l_run;   // this lane's partial sum of P (its half of the keys)
};

// S^T = K' Q'^T for one 32-key block.  Lane (q = l%32, h = l/32): register r
// holds key kblk + 8 (r/4) + 4 h + r%4.  kblk_lds points at the block's first
// K' row in LDS; kread_off is this lane's swizzled offset of row q%32, chunk
// 8h, and k-step kk is reached by XOR with kk << 4.
__device__ __forceinline__ void qk_blk(f32x16& s, const lds_u8* kblk_lds, uint32_t kread_off,
                                       const bf16x8 (&qf)[8]) {
  s = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 a = lds_read_b128(kblk_lds + (kread_off ^ (uint32_t)(kk << 4)));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
  }
}

// Masked-out keys -> -inf: visible iff 0 <= qm - key < lim.
__device__ __forceinline__ void mask_blk(f32x16& s, int kblk, int qm, int lim, int half) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int dq = qm - (kblk + 8 * (r >> 2) + 4 * half + (r & 3));
    s[r] = (unsigned)dq < (unsigned)lim ? s[r] : -INFINITY;
  }
}

// Row max of the raw scores of one block (both lane halves of the row).
__device__ __forceinline__ float blk_max(const f32x16& s) {
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
  return pair_max32(mx);
}

// Running max update with lazy rescaling of the accumulator; returns -m*c.
__device__ __forceinline__ float softmax_rescale(TileState& st, float mx, float c,
                                                 float rescale_raw) {
  const float m_new = fmaxf(st.m_run, mx);
  if (__builtin_amdgcn_ballot_w64(m_new > st.m_run + rescale_raw)) {
    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2((st.m_run - m_new) * c);
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) st.acc[bd] *= alpha;
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  return st.m_run == -INFINITY ? 0.0f : -st.m_run * c;
}

// P = exp2(s c - m c) packed to bf16 (the PV B operand for the block's two
// 16-key k-steps), row sums from the rounded values the MFMA multiplies.
__device__ __forceinline__ void exp_blk(TileState& st, const f32x16& s, float c, float neg_mc,
                                        bf16x8 (&pf)[2]) {
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(s[8 * t + e], c, neg_mc));
    pf[t] = pack_bf16x8(pv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 pr = {pf[t][2 * e], pf[t][2 * e + 1]};
      st.l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, st.l_run, false);
    }
  }
}

// O^T += V^T P^T for one 32-key block.  k-step t covers keys 16t .. 16t+15 of
// the block; this lane half supplies keys 4h+0..3 (first transposing load)
// and 8+4h+0..3.  O^T register r of block bd holds dim 32 bd + 8 (r/4) + 4 h
// + r%4.  vread[bd]: this lane's swizzled address for dim block bd in the
// block's V row 4h + i/4 (i = lane % 16).
__device__ __forceinline__ void pv_blk(TileState& st, const lds_u8* (&vread)[4], int row0,
                                       const bf16x8 (&pf)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      const lds_u8* p0 = vread[bd] + (row0 + 16 * t) * kRowBytes;
      const bf16x8 a = lds_read_tr2(p0, p0 + 8 * kRowBytes);
      st.acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[t], st.acc[bd], 0, 0, 0);
    }
  }
}

// Split forms of qk_blk / pv_blk for the software-pipelined global loop: the
// LDS operand reads are issued early, into registers, and the MFMAs run
// back to back once they have landed.
__device__ __forceinline__ void load_kops(bf16x8 (&ka)[8], const lds_u8* kblk_lds, uint32_t kread_off) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) ka[kk] = lds_read_b128(kblk_lds + (kread_off ^ (uint32_t)(kk << 4)));
}

__device__ __forceinline__ void qk_mfma(f32x16& s, const bf16x8 (&ka)[8], const bf16x8 (&qf)[8]) {
  s = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s, 0, 0, 0);
}

// va[4 t + bd]: the A operand of k-step t, dim block bd
__device__ __forceinline__ void load_vops(bf16x8 (&va)[8], const lds_u8* const (&vread)[4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      const lds_u8* p0 = vread[bd] + 16 * t * kRowBytes;
      va[4 * t + bd] = lds_read_tr2(p0, p0 + 8 * kRowBytes);
    }
  }
}

// Query normalisation of one lane: x holds dims 64 half .. 64 half + 63 of
// its raw query row.  RMSNorm over the 128 dims (both lane halves), the
// weight, then the partial rotation at position pos (rotary pairs (t, t +
// R/2), all inside lane half 0); x then holds those dims of q'.  RH:
// rope_dim / 2 when fixed at compile time (21 or 0: the rotation stays in
// registers); -1 for any other even rope_dim <= 64, which rotates through
// qs, a private LDS row of 64 floats of this lane.  qw: the 128 query-norm
// weights (p.q_norm_w, or a copy of them in LDS).
template <int RH>
__device__ __forceinline__ void q_norm_rope(float (&x)[64], int half, const FlashParams& p,
                                            long long pos, float* qs, const float* qw) {
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < 64; ++d) ss += x[d] * x[d];
  ss = pair_sum32(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
  const float* wsrc = qw + 64 * half;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    u32x4 wv4 = ld16(wsrc + 4 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * j + i] *= r * __uint_as_float(wv4[i]);
  }
  if (RH > 0 && half == 0) {
    float y[2 * (RH > 0 ? RH : 1)];
#pragma unroll
    for (int t = 0; t < RH; ++t) {
      float cc, sn;
      rope_cos_sin(p.tab, t, pos, cc, sn);
      y[t] = x[t] * cc - x[t + RH] * sn;
      y[t + RH] = x[t + RH] * cc + x[t] * sn;
    }
#pragma unroll
    for (int d = 0; d < 2 * RH; ++d) x[d] = y[d];
  } else if (RH < 0 && p.rope_half > 0 && half == 0) {
#pragma unroll
    for (int d = 0; d < 64; ++d) qs[d] = x[d];
    const int rh = p.rope_half;
#pragma unroll
    for (int t = 0; t < kMaxRopeHalf; ++t) {
      if (t < rh) {
        float cc, sn;
        rope_cos_sin(p.tab, t, pos, cc, sn);
        const float a = qs[t], bb = qs[t + rh];
        qs[t] = a * cc - bb * sn;
        qs[t + rh] = bb * cc + a * sn;
      }
    }
#pragma unroll
    for (int d = 0; d < 64; ++d) x[d] = qs[d];
  }
}

// The query prologue of the bf16 kernels: q' times c = softmax scale *
// log2(e), packed as the 8 k-steps of the score products' B operand (the
// products then come out in exp2 units).
template <int RH>
__device__ __forceinline__ void q_prologue(float (&x)[64], int half, const FlashParams& p,
                                           long long pos, float* qs, bf16x8 (&qf)[8],
                                           const float* qw) {
  q_norm_rope<RH>(x, half, p, pos, qs, qw);
#pragma unroll
  for (int d = 0; d < 64; ++d) x[d] *= p.scale_log2;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = pack_bf16x8(x + 8 * kk);
}

}  // namespace flash
}  // namespace zg
