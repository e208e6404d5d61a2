// Training backward of the gated sliding-window / global attention layer.
//
// The pages measure the model in training (page "ZGCM-1:面向数学与智能体搜索的全
// 开源高效基础模型", section 前置知识 and the architecture ablation; page "7B 打
// 235B？…全开源配方", section 🏗️ 架构) but define only the forward pass: QK-RMSNorm,
// partial RoPE, softmax attention over the causal band (128 keys) or the
// whole causal prefix, GQA with 4 query heads per KV head, and a sigmoid gate
// on the windowed layers' output.  What follows is that forward's derivative,
// for L = sum(dY * Y):
//
//   sig = sigmoid(G);  dO = dY * sig;  dG = dY * Y * (1 - sig)   (Y = O * sig)
//   Dr_i = sum_d dO_id O_id = sum_d dY_id Y_id
//   P = exp(tau q'k'^T - LSE);  dP = dO V^T;  dS = P * (dP - Dr)
//   dq' = tau dS K';  dk'_g = tau sum_h dS_h^T Q'_h;  dv_g = sum_h P_h^T dO_h
//   then back through the RoPE rotation (its transpose) and RMSNorm.
//
// Kernels:
//   bwd_prep_kernel      dO, dG, Dr and LSE*log2(e) per query row
//   bwd_dq_kernel        query-stationary: dq' for 32 rows per wave; K' and V
//                        tiles stream through LDS as in the forward; forms
//                        Q' from q itself (rope_dim 42 or 0) and writes it
//   bwd_dkv_kernel       key-stationary: dk' and dv for 32 keys per wave,
//                        summed over the group's query heads; Q' and dO
//                        tiles stream through LDS
//   prologue_bwd_kernel  RoPE transpose + RMSNorm backward per row, and
//                        per-block partial sums of the weight gradient
// Splitting dq' from dk'/dv (each kernel recomputes P) avoids atomics.
//
// Tiles in LDS are 32 rows of 256 bytes whose 16-byte chunks are permuted by
// row: physical chunk = logical ^ swz(row), swz(row) = (row & 3) << 2 |
// (row >> 2) & 3.  Rows 0..15 get 16 distinct values, so a 16-lane
// ds_read_b128 of one logical chunk from 16 rows is conflict-free; the four
// rows 4n..4n+3 of a transposing read get values that differ in bits 2-3,
// so ds_read_b64_tr_b16 of two adjacent chunks per row is conflict-free too.

#include "zg_common.h"
#include "zg_launch.h"
#include "zg_lds.h"

namespace zg {

namespace {

constexpr int kRowB = kD * 2;       // 256-byte bf16 rows
constexpr int kTileB = 32 * kRowB;  // 32-row tile, 8 KB

__device__ __forceinline__ uint32_t swz(int row) {
  return (uint32_t)(((row & 3) << 2) | ((row >> 2) & 3));
}

// Per-lane offsets of the transposing reads that form an MFMA A operand
// (32 dims x 16 rows, dims = l % 32 within block bd, rows of k-step t) from
// a swizzled 32-row tile.  Lane l: 16-lane group G = l / 16, i = l % 16;
// the first load covers rows 16t + 4(G/2) + 0..3, the second rows 8 further.
struct TrOffsets {
  uint32_t off[4];  // dim block bd, first load, k-step 0
  int delta;        // second load relative to the first
};

__device__ __forceinline__ TrOffsets tr_offsets(int lane) {
  TrOffsets o;
  const int G = lane >> 4, i = lane & 15;
  const int hq = G >> 1, vq = i >> 2;
  const int lo2 = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
    o.off[bd] = (uint32_t)((4 * hq + vq) * kRowB + ((((bd ^ vq) << 2) | (lo2 ^ hq)) << 4) + 8 * (i & 1));
  o.delta = 8 * kRowB + (((lo2 ^ hq) & 2) ? -32 : 32);
  return o;
}

__device__ __forceinline__ bf16x8 tr_operand(const lds_u8* tile, const TrOffsets& o, int bd, int t) {
  const lds_u8* p0 = tile + o.off[bd] + t * 16 * kRowB;
  return lds_read_tr2(p0, p0 + o.delta);
}

// ---------------------------------------------------------------------------
// Per query row (b, s, h): Dr = sum dY*Y, dO = dY*sig(G), dG = dY*Y*(1-sig(G)),
// lse2 = LSE*log2(e).  Rows are enumerated over (b, h, s < Spad); rows past S
// get lse2 = +inf and Dr = 0, so that they contribute P = 0 downstream.
// 16 lanes per row, 8 dims each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ dy,
                                                       const uint16_t* __restrict__ y,
                                                       const uint16_t* __restrict__ gate,
                                                       const float* __restrict__ lse,
                                                       uint16_t* __restrict__ dO,
                                                       uint16_t* __restrict__ dgate,
                                                       float* __restrict__ lse2,
                                                       float* __restrict__ dvec, int B, int S,
                                                       int Spad, int Hq) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c16 = threadIdx.x & 15;
  if (row >= (long long)B * Hq * Spad) return;  // whole 16-lane groups leave together
  const int s = (int)(row % Spad);
  const long long bh = row / Spad;
  if (s >= S) {
    if (c16 == 0) {
      lse2[row] = INFINITY;
      dvec[row] = 0.f;
    }
    return;
  }
  const int h = (int)(bh % Hq);
  const long long b = bh / Hq;
  const long long off = ((b * S + s) * Hq + h) * kD + 8 * c16;
  float fy[8], fo[8];
  unpack_bf16x8(ld16(dy + off), fy);
  unpack_bf16x8(ld16(y + off), fo);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) d += fy[e] * fo[e];
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) d += __shfl_xor(d, m, 16);
  if (gate) {
    float fg[8], od[8], gd[8];
    unpack_bf16x8(ld16(gate + off), fg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = sigmoidf_(fg[e]);
      od[e] = fy[e] * sg;
      gd[e] = fy[e] * fo[e] * (1.0f - sg);
    }
    u32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = pack_bf16x2(od[2 * e], od[2 * e + 1]);
      w1[e] = pack_bf16x2(gd[2 * e], gd[2 * e + 1]);
    }
    st16(dO + off, w0);
    st16(dgate + off, w1);
  }
  if (c16 == 0) {
    lse2[row] = lse[bh * S + s] * kLog2e;
    dvec[row] = d;
  }
}

// ---------------------------------------------------------------------------
// dq': one 256-thread workgroup = (batch, kv head g, block of query
// positions), its 4 waves the group's query heads (as in the forward).  Per
// 32-key tile and wave:
//   S^T  = K' Q'^T   (A = K' rows, ds_read_b128; B = Q' in registers)
//   dP^T = V dO^T    (A = V rows, ds_read_b128; B = dO in registers)
//   P^T = exp2(S^T c - lse2), dS^T = P^T (dP^T - Dr)
//   dQ^T += K'^T dS^T (A = K'^T by transposing reads; B = dS^T as bf16)
// K'/V tiles come through a three-stage ring of untracked copies.
// ---------------------------------------------------------------------------
struct DqGeo {
  int hpw;  // query heads per workgroup
  int ppw;  // query positions per workgroup
  int n_pos_blocks, hgroups, n_bhg;
};

// RH = rope_dim / 2 when Q' is formed here (21 or 0), -1 when it is read
// from p.qp.
template <int RH>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p, DqGeo geo) {
  constexpr int NS = 3;
  constexpr int kVOff = NS * kTileB;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * NS * kTileB];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int qcol = lane & 31, half = lane >> 5;
  const int grp = p.Hq / p.Hkv;
  const bool banded = p.window > 0;

  const int bid = blockIdx.x;
  const int bhg = bid % geo.n_bhg;
  int pb = bid / geo.n_bhg;
  if (!banded) pb = geo.n_pos_blocks - 1 - pb;  // longest causal rows first
  const int hg = bhg % geo.hgroups;
  const int bgi = bhg / geo.hgroups;
  const int g = bgi % p.Hkv;
  const int b = bgi / p.Hkv;
  const int head = g * grp + hg * geo.hpw + (wvu % geo.hpw);
  const int i0w = pb * geo.ppw;
  const int wrow0 = i0w + (wvu / geo.hpw) * 32;
  const int qi = wrow0 + qcol;
  const bool qok = qi < p.S;
  const int lim = banded ? p.window : 0x7fffffff;
  const int hi = min(p.S, i0w + geo.ppw);
  const int lo = banded ? max(0, i0w - p.window + 1) : 0;
  const int t_hi = (hi - 1) / 32;
  const int nt = t_hi - lo / 32 + 1;

  // ---- K'/V tile copies: wave w fills 1 KB blocks 2w, 2w+1 of each tile
  const long long kvstride = (long long)p.Hkv * kD;
  const uint16_t* kbase = p.kp + (long long)b * p.S * kvstride + g * kD;
  const uint16_t* vbase = p.v + (long long)b * p.S * kvstride + g * kD;
  uint32_t row_off[2], chk[2];
  int lrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lrow[j] = 4 * (2 * wvu + j) + (lane >> 4);
    row_off[j] = (uint32_t)(lrow[j] * kvstride * 2);
    chk[j] = 16u * ((uint32_t)(lane & 15) ^ swz(lrow[j]));
  }
  auto gload = [&](int t, int stg) {
    const unsigned char* kb = (const unsigned char*)(kbase + (long long)t * 32 * kvstride);
    const unsigned char* vb = (const unsigned char*)(vbase + (long long)t * 32 * kvstride);
    const uint32_t kl = lds_addr(smem + stg * kTileB + 2 * wvu * 1024);
    const uint32_t vl = kl + kVOff;
    if (t * 32 + 32 <= p.S) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dma16_s(kb, row_off[j] + chk[j], kl + j * 1024);
        dma16_s(vb, row_off[j] + chk[j], vl + j * 1024);
      }
    } else {  // keys past S (top tile only) read key S-1; they are masked
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t off = (uint32_t)((min(t * 32 + lrow[j], p.S - 1) - t * 32) * kvstride * 2);
        dma16_s(kb, off + chk[j], kl + j * 1024);
        dma16_s(vb, off + chk[j], vl + j * 1024);
      }
    }
  };
  gload(t_hi, 0);
  if (nt > 1) gload(t_hi - 1, 1);

  // ---- this lane's query row: Q' and dO as B operands, lse2 and Dr
  const long long qrow = ((long long)b * p.S + (qok ? qi : 0)) * p.Hq + head;
  bf16x8 qf[8], of[8];
  {
    const uint16_t* os = p.dO + qrow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      of[j] = __builtin_bit_cast(bf16x8, qok ? ld16(os + 8 * j) : u32x4{0, 0, 0, 0});
    if constexpr (RH >= 0) {
      // Q' of this lane's half row: RMSNorm (+ weight) and the rotary pairs
      // (t, t + RH), with the same expressions in the same order as the
      // forward's fused query prologue, so that these are the bits the
      // forward multiplied.  Written to p.qp for the dk'/dv kernel.
      const uint16_t* src = p.q + qrow * kD + 64 * half;
      float x[64];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 u = qok ? ld16(src + 8 * j) : u32x4{0, 0, 0, 0};
        unpack_bf16x8(u, x + 8 * j);
      }
      float ss = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) ss += x[d] * x[d];
      ss = pair_sum32(ss);
      const float r = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
      const float* wsrc = p.q_norm_w + 64 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const u32x4 w4 = ld16(wsrc + 4 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * j + i] *= r * __uint_as_float(w4[i]);
      }
      if (RH > 0 && half == 0) {
        const long long pos = p.pos_offset + qi;
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
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qf[kk] = pack_bf16x8(x + 8 * kk);
      if (qok) {
        uint16_t* dst = const_cast<uint16_t*>(p.qp) + qrow * kD + 64 * half;
#pragma unroll
        for (int j = 0; j < 8; ++j) st16(dst + 8 * j, __builtin_bit_cast(u32x4, qf[j]));
      }
    } else {
      const uint16_t* qs = p.qp + qrow * kD + 64 * half;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qf[j] = __builtin_bit_cast(bf16x8, qok ? ld16(qs + 8 * j) : u32x4{0, 0, 0, 0});
    }
  }
  const long long lrw = ((long long)b * p.Hq + head) * p.Spad + qi;  // qi < Spad
  const float lse_l = p.lse2[lrw];
  const float d_l = p.dvec[lrw];
  const float c = p.scale_log2;

  const uint32_t bread = (uint32_t)qcol * kRowB + (((uint32_t)(8 * half) ^ swz(qcol)) << 4);
  const TrOffsets tro = tr_offsets(lane);

  f32x16 acc[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) acc[bd] = f32x16{};

  if (nt > 1) sync_tiles<4>();
  else sync_tiles<0>();

  int stg = 0;
  for (int j = 0; j < nt; ++j) {
    const int t = t_hi - j;
    const bool issue = j + 2 < nt;
    if (issue) gload(t - 2, stg == 0 ? 2 : stg - 1);
    const lds_u8* kt = smem + stg * kTileB;
    const lds_u8* vt = kt + kVOff;
    f32x16 sT = f32x16{}, dpT = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kt + (bread ^ (uint32_t)(kk << 4))),
                                                   qf[kk], sT, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      dpT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(vt + (bread ^ (uint32_t)(kk << 4))),
                                                    of[kk], dpT, 0, 0, 0);
    // register r: key t*32 + 8(r/4) + 4 half + r%4 of this lane's query
    const bool masked = banded || t * 32 + 31 > wrow0;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = fast_exp2(__builtin_fmaf(sT[r], c, -lse_l));
      if (masked) {
        const int dq = qi - (t * 32 + 8 * (r >> 2) + 4 * half + (r & 3));
        pr = (unsigned)dq < (unsigned)lim ? pr : 0.f;
      }
      ds[r] = pr * (dpT[r] - d_l);
    }
    const bf16x8 dsf0 = pack_bf16x8(ds), dsf1 = pack_bf16x8(ds + 8);
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
      acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kt, tro, bd, 0), dsf0, acc[bd], 0, 0, 0);
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
      acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kt, tro, bd, 1), dsf1, acc[bd], 0, 0, 0);
    // tile j+1 must have landed; tile j+2's four copies may still fly
    if (issue) sync_tiles<4>();
    else sync_tiles<0>();
    stg = stg == 2 ? 0 : stg + 1;
  }

  // dq' = tau * dQ; register r of block bd -> dim 32bd + 8(r/4) + 4 half + r%4
  if (qok) {
    uint16_t* dst = p.dqp + qrow * kD + 4 * half;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& a = acc[bd];
        uint2 w;
        w.x = pack_bf16x2(a[4 * q4] * p.scale, a[4 * q4 + 1] * p.scale);
        w.y = pack_bf16x2(a[4 * q4 + 2] * p.scale, a[4 * q4 + 3] * p.scale);
        *reinterpret_cast<uint2*>(dst + 32 * bd + 8 * q4) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dk' and dv: one 256-thread workgroup = (batch, kv head g, block of 128
// keys), wave w owning keys 32w..32w+31 of the block.  The workgroup visits
// every (query head of the group, 32-query tile) whose queries can see its
// keys: query tiles from the last one down, the group's heads innermost.
// Workgroups of one KV head that run at the same time (consecutive key
// blocks, on one XCD) then read the same Q'/dO tiles at about the same time,
// out of that XCD's L2.  Per tile and wave, with this lane's key in column
// l % 32:
//   S  = Q' K'^T  (A = Q' rows, ds_read_b128; B = K' in registers)
//   dP = dO V^T   (A = dO rows; B = V rows of the block, both ds_read_b128)
//   P = exp2(S c - lse2), dS = P (dP - Dr)
//   dV^T += dO^T P, dK^T += Q'^T dS  (A by transposing reads; B = P, dS)
// The block's V rows sit in LDS for the whole kernel (keeping them in
// registers would leave room for one wave per SIMD only); Q'/dO tiles and
// the tile's lse2 / Dr come through a two-stage ring of untracked copies
// (five per wave and tile).
// ---------------------------------------------------------------------------
constexpr int kDkvStage = 2 * kTileB + 256;  // Q', dO, lse2[32], Dr[32]
constexpr int kDkvV = 2 * kDkvStage;         // V rows of the key block, 4 x 8 KB

__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * kDkvStage + 4 * kTileB];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int qcol = lane & 31, half = lane >> 5;
  const int grp = p.Hq / p.Hkv;
  const bool banded = p.window > 0;
  const int lim = banded ? p.window : 0x7fffffff;

  const int bid = blockIdx.x;
  const int bg = bid % (p.B * p.Hkv);
  const int kb = bid / (p.B * p.Hkv);  // key block 0 (most queries) first
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int kb0 = kb * 128;
  const int kj = kb0 + 32 * wvu + qcol;  // this lane's key
  const bool kok = kj < p.S;

  // query tiles whose queries can see some key of the block
  const int qt_lo = kb0 / 32;
  const int q_last = banded ? min(p.S - 1, kb0 + 127 + p.window - 1) : p.S - 1;
  const int nq = q_last / 32 - qt_lo + 1;
  const int ntile = grp * nq;

  // ---- copies: Q' / dO rows 4(2w+j) + L/16 of the tile; lse2 / Dr: lanes
  // 0..3 of each wave, 16 floats per wave
  const long long qstride = (long long)p.Hq * kD;  // elements between query rows
  int lrow[2];
  uint32_t chk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lrow[j] = 4 * (2 * wvu + j) + (lane >> 4);
    chk[j] = 16u * ((uint32_t)(lane & 15) ^ swz(lrow[j]));
  }
  auto gload = [&](int i, int stg) {
    const int hh = i % grp;
    const int q0 = (qt_lo + nq - 1 - i / grp) * 32;
    const int head = g * grp + hh;
    const long long base = ((long long)b * p.S + q0) * qstride + (long long)head * kD;
    const unsigned char* qb = (const unsigned char*)(p.qp + base);
    const unsigned char* ob = (const unsigned char*)(p.dO + base);
    const uint32_t sb = lds_addr(smem + stg * kDkvStage);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // rows past S read row S-1 (their lse2 is +inf, so P = 0)
      const uint32_t off = (uint32_t)((min(q0 + lrow[j], p.S - 1) - q0) * qstride * 2) + chk[j];
      dma16_s(qb, off, sb + (2 * wvu + j) * 1024);
      dma16_s(ob, off, sb + kTileB + (2 * wvu + j) * 1024);
    }
    const long long vrow = ((long long)b * p.Hq + head) * p.Spad + q0;
    if (lane < 4) {
      const float* src = (wvu < 2 ? p.lse2 : p.dvec) + vrow + 16 * (wvu & 1) + 4 * lane;
      dma16(src, sb + 2 * kTileB + 64 * wvu);
    }
  };
  // ---- the wave's 32 V rows -> LDS (8 copies of 1 KB: rows 4n + L/16 of
  // its slice, swizzled; rows past S read row S-1 and are never visible)
  {
    const long long vstride = (long long)p.Hkv * kD;
    const int r0 = kb0 + 32 * wvu;
    const unsigned char* vb =
        (const unsigned char*)(p.v + ((long long)b * p.S + min(r0, p.S - 1)) * vstride + g * kD);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int rl = 4 * n + (lane >> 4);  // row within the wave's slice
      const uint32_t off = (uint32_t)((min(r0 + rl, p.S - 1) - min(r0, p.S - 1)) * vstride * 2) +
                           16u * ((uint32_t)(lane & 15) ^ swz(rl));
      dma16_s(vb, off, lds_addr(smem + kDkvV + wvu * kTileB + n * 1024));
    }
  }
  gload(0, 0);
  if (ntile > 1) gload(1, 1);

  // ---- this lane's key: K' as the B operand (dims 64 half + 8kk ..)
  bf16x8 kf[8];
  {
    const long long krow = ((long long)b * p.S + (kok ? kj : 0)) * p.Hkv + g;
    const uint16_t* ks = p.kp + krow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      kf[j] = __builtin_bit_cast(bf16x8, kok ? ld16(ks + 8 * j) : u32x4{0, 0, 0, 0});
  }
  const lds_u8* vblk = smem + kDkvV + wvu * kTileB;  // this wave's V rows
  const float c = p.scale_log2;
  const uint32_t bread = (uint32_t)qcol * kRowB + (((uint32_t)(8 * half) ^ swz(qcol)) << 4);
  const TrOffsets tro = tr_offsets(lane);

  f32x16 dk[4], dvv[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) {
    dk[bd] = f32x16{};
    dvv[bd] = f32x16{};
  }

  if (ntile > 1) sync_tiles<5>();
  else sync_tiles<0>();

  for (int i = 0; i < ntile; ++i) {
    const int stg = i & 1;
    const int q0 = (qt_lo + nq - 1 - i / grp) * 32;
    const lds_u8* qt = smem + stg * kDkvStage;
    const lds_u8* ot = qt + kTileB;
    const lds_u8* lt = qt + 2 * kTileB;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(qt + (bread ^ (uint32_t)(kk << 4))),
                                                  kf[kk], s, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(ot + (bread ^ (uint32_t)(kk << 4))),
                                                   lds_read_b128(vblk + (bread ^ (uint32_t)(kk << 4))),
                                                   dp, 0, 0, 0);
    // register r: query q0 + 8(r/4) + 4 half + r%4, key kj
    float pr[16], ds[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 l4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          lt + 4 * (8 * m + 4 * half));
      const f32x4 d4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          lt + 128 + 4 * (8 * m + 4 * half));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * m + e;
        const int dq = q0 + 8 * m + 4 * half + e - kj;
        float x = fast_exp2(__builtin_fmaf(s[r], c, -l4[e]));
        x = (unsigned)dq < (unsigned)lim ? x : 0.f;
        pr[r] = x;
        ds[r] = x * (dp[r] - d4[e]);
      }
    }
    const bf16x8 pf0 = pack_bf16x8(pr), pf1 = pack_bf16x8(pr + 8);
    const bf16x8 df0 = pack_bf16x8(ds), df1 = pack_bf16x8(ds + 8);
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      dvv[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(ot, tro, bd, 0), pf0, dvv[bd], 0, 0, 0);
      dk[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(qt, tro, bd, 0), df0, dk[bd], 0, 0, 0);
    }
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      dvv[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(ot, tro, bd, 1), pf1, dvv[bd], 0, 0, 0);
      dk[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(qt, tro, bd, 1), df1, dk[bd], 0, 0, 0);
    }
    // tile i+1 has landed and every wave is done with tile i; then tile i+2
    // goes into tile i's stage
    sync_tiles<0>();
    if (i + 2 < ntile) gload(i + 2, stg);
  }

  // register r of block bd -> dim 32bd + 8(r/4) + 4 half + r%4 of key kj
  if (kok) {
    const long long krow = ((long long)b * p.S + kj) * p.Hkv + g;
    uint16_t* dkd = p.dkp + krow * kD + 4 * half;
    uint16_t* dvd = p.dv + krow * kD + 4 * half;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 k2;
        k2.x = pack_bf16x2(dk[bd][4 * q4] * p.scale, dk[bd][4 * q4 + 1] * p.scale);
        k2.y = pack_bf16x2(dk[bd][4 * q4 + 2] * p.scale, dk[bd][4 * q4 + 3] * p.scale);
        *reinterpret_cast<uint2*>(dkd + 32 * bd + 8 * q4) = k2;
        uint2 w;
        w.x = pack_bf16x2(dvv[bd][4 * q4], dvv[bd][4 * q4 + 1]);
        w.y = pack_bf16x2(dvv[bd][4 * q4 + 2], dvv[bd][4 * q4 + 3]);
        *reinterpret_cast<uint2*>(dvd + 32 * bd + 8 * q4) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Back through RoPE and RMSNorm, per row of `heads` heads (16 lanes x 8 dims):
//   dx_hat = R(-phi) dy'               (transpose of the rotary pairs)
//   r = (mean(x^2) + eps)^-1/2
//   dx = r (w * dx_hat) - x r^3 mean(w * dx_hat * x)
//   dw += dx_hat * x * r              (per-block partials, summed later)
// A fixed grid of kBwdParts blocks (eight per CU; at 87 VGPRs five are
// resident at a time) strides over groups of 16 rows; each group's x and dy'
// rows are loaded one iteration ahead, and the barriers wait for LDS only, so
// those loads stay in flight across them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prologue_bwd_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ dyp,
                                                           const float* __restrict__ w,
                                                           uint16_t* __restrict__ dx,
                                                           float* __restrict__ part, long long rows,
                                                           int S, int heads, long long pos_offset,
                                                           int rope_half, float eps, RopeTable tab) {
  __shared__ float rowbuf[16][kD + 4];
  __shared__ float cs[16][kMaxRopeHalf], sn[16][kMaxRopeHalf];
  const int slot = threadIdx.x >> 4, c16 = threadIdx.x & 15;
  float wl[8];
  {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + 8 * c16);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + 8 * c16 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wl[e] = w0[e];
      wl[4 + e] = w1[e];
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int R = 2 * rope_half;
  if (rows == 0) {
    if (threadIdx.x < kD) part[(long long)blockIdx.x * kD + threadIdx.x] = 0.f;
    return;
  }
  // Rows past the end read row rows - 1 (always in bounds, no branch, so the
  // next group's loads need no wait before this group's work) and store
  // nothing; an in-range row reads no other slot's row or angles.
  auto load = [&](long long rg, u32x4& xu, u32x4& du) {
    const long long row = min(rg * 16 + slot, rows - 1);
    xu = ld16(x + row * kD + 8 * c16);
    du = ld16(dyp + row * kD + 8 * c16);
  };
  // this lane's rotary frequencies (angles t = c16 and c16 + 16; rope_half <= 32)
  static_assert(kMaxRopeHalf <= 32, "two angles per lane");
  const uint64_t fr0 = c16 < rope_half ? tab.frac[c16] : 0;
  const uint64_t fr1 = c16 + 16 < rope_half ? tab.frac[c16 + 16] : 0;
  u32x4 xu, du;
  load(blockIdx.x, xu, du);
  for (long long rg = blockIdx.x; rg * 16 < rows; rg += gridDim.x) {  // uniform per block
    const long long row = rg * 16 + slot;
    const bool ok = row < rows;
    float xv[8], dyv[8];
    unpack_bf16x8(xu, xv);
    unpack_bf16x8(du, dyv);
    load(rg + gridDim.x, xu, du);  // the next group's rows
    const long long pos = pos_offset + (row / heads) % S;
    if (R > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rowbuf[slot][8 * c16 + e] = dyv[e];
      // the block's first row of each position computes its angles, one per
      // lane t % 16, for all rows of that position
      if ((int)(row % heads) == 0 || slot == 0) {
        if (c16 < rope_half) rope_cos_sin_f(fr0, pos, cs[slot][c16], sn[slot][c16]);
        if (c16 + 16 < rope_half) rope_cos_sin_f(fr1, pos, cs[slot][c16 + 16], sn[slot][c16 + 16]);
      }
    }
    lds_barrier();
    const int ref = slot - (int)min(row % heads, (long long)slot);
    float dh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * c16 + e;
      dh[e] = dyv[e];
      if (d < R) {
        const int t = d < rope_half ? d : d - rope_half;
        const float c = cs[ref][t], s = sn[ref][t];
        if (d < rope_half) dh[e] = dyv[e] * c + rowbuf[slot][d + rope_half] * s;
        else dh[e] = dyv[e] * c - rowbuf[slot][d - rope_half] * s;
      }
    }
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += xv[e] * xv[e];
      dot += wl[e] * dh[e] * xv[e];
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      ss += __shfl_xor(ss, m, 16);
      dot += __shfl_xor(dot, m, 16);
    }
    const float r = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
    const float k3 = r * r * r * dot * (1.0f / kD);
    if (ok) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = r * wl[e] * dh[e] - xv[e] * k3;
        acc[e] += dh[e] * xv[e] * r;
      }
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
      st16(dx + row * kD + 8 * c16, u);
    }
    lds_barrier();  // rowbuf and the angle tables are rewritten by the next group
  }
  // sum the 16 row slots of the block
#pragma unroll
  for (int e = 0; e < 8; ++e) rowbuf[slot][8 * c16 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < kD) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += rowbuf[k][threadIdx.x];
    part[(long long)blockIdx.x * kD + threadIdx.x] = s;
  }
}

// dw[d] = sum over the kBwdParts partials in a fixed order (deterministic):
// thread (chunk c, dim d) sums partials c*kChunk .. c*kChunk + kChunk - 1 in
// order, then the eight chunk sums are added in order of c.
constexpr int kReduceChunks = 8;
__global__ __launch_bounds__(kReduceChunks * kD) void reduce_parts_kernel(const float* __restrict__ part,
                                                                          float* __restrict__ dw) {
  constexpr int kChunk = kBwdParts / kReduceChunks;
  __shared__ float red[kReduceChunks][kD];
  const int d = threadIdx.x % kD, c = threadIdx.x / kD;
  const float* src = part + (long long)c * kChunk * kD + d;
  float s = 0.f;
#pragma unroll 16
  for (int k = 0; k < kChunk; ++k) s += src[(long long)k * kD];
  red[c][d] = s;
  __syncthreads();
  if (c == 0) {
    float t = red[0][d];
#pragma unroll
    for (int j = 1; j < kReduceChunks; ++j) t += red[j][d];
    dw[d] = t;
  }
}
static_assert(kBwdParts % kReduceChunks == 0, "partials split evenly over the chunks");

}  // namespace

hipError_t launch_bwd_prep(const uint16_t* dy, const uint16_t* y, const uint16_t* gate,
                           const float* lse, uint16_t* dO, uint16_t* dgate, float* lse2,
                           float* dvec, int B, int S, int Spad, int Hq, hipStream_t stream) {
  const long long rows = (long long)B * Hq * Spad;
  if (rows == 0) return hipSuccess;
  const long long blocks = (rows + 15) / 16;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dy, y, gate, lse,
                     dO, dgate, lse2, dvec, B, S, Spad, Hq);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const int grp = p.Hq / p.Hkv;
  DqGeo geo;
  geo.hpw = grp < 4 ? grp : 4;
  geo.hgroups = grp / geo.hpw;
  geo.ppw = 128 / geo.hpw;
  geo.n_pos_blocks = (p.S + geo.ppw - 1) / geo.ppw;
  geo.n_bhg = p.B * p.Hkv * geo.hgroups;
  const long long blocks = (long long)geo.n_pos_blocks * geo.n_bhg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (!bwd_dq_fuses_q(p.rope_half))
    hipLaunchKernelGGL(bwd_dq_kernel<-1>, dim3((unsigned)blocks), dim3(256), 0, stream, p, geo);
  else if (p.rope_half == 21)
    hipLaunchKernelGGL(bwd_dq_kernel<21>, dim3((unsigned)blocks), dim3(256), 0, stream, p, geo);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, p, geo);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const long long blocks = (long long)((p.S + 127) / 128) * p.B * p.Hkv;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prologue_bwd(const uint16_t* x, const uint16_t* dyp, const float* w, uint16_t* dx,
                               float* part, long long rows, int S, int heads, long long pos_offset,
                               int rope_half, float eps, const RopeTable& tab, hipStream_t stream) {
  hipLaunchKernelGGL(prologue_bwd_kernel, dim3(kBwdParts), dim3(256), 0, stream, x, dyp, w, dx, part,
                     rows, S, heads, pos_offset, rope_half, eps, tab);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(const float* part, float* dw, hipStream_t stream) {
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(1), dim3(kReduceChunks * kD), 0, stream, part, dw);
  return hipGetLastError();
}

}  // namespace zg
