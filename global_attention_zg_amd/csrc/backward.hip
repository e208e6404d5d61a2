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
//                        Q' from q itself (rope_dim 42 or 0) and writes it;
//                        then back through RoPE and RMSNorm to dq
//   bwd_dkv_kernel       key-stationary: dk' and dv for 32 keys per wave,
//                        summed over the group's query heads; Q' and dO
//                        tiles stream through LDS; then dk' back to dk
//   reduce_*_kernel      the norm-weight gradients from one partial sum per
//                        workgroup of the two kernels above, in a fixed order
// Splitting dq' from dk'/dv (each kernel recomputes P) avoids atomics.
//
// Tiles in LDS are 32 rows of 256 bytes whose 16-byte chunks are permuted by
// row: physical chunk = logical ^ swz(row), swz(row) = (row & 3) << 2 |
// (row >> 2) & 3.  Rows 0..15 get 16 distinct values, so a 16-lane
// ds_read_b128 of one logical chunk from 16 rows is conflict-free; the four
// rows 4n..4n+3 of a transposing read get values that differ in bits 2-3,
// so ds_read_b64_tr_b16 of two adjacent chunks per row is conflict-free too.

#include <type_traits>

#include "zg_common.h"
#include "zg_launch.h"
#include "zg_lds.h"
#include "zg_norm_rope.h"

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
// Back through RoPE and RMSNorm, for the 32 rows one wave owns (one head,
// consecutive positions pos0, pos0 + 1, ...), 16 lanes per row and 8 dims per
// lane, four rows per pass:
//   dx_hat = R(-phi) dy'               (transpose of the rotary pairs)
//   r = (mean(x^2) + eps)^-1/2
//   dx = r (w * dx_hat) - x r^3 mean(w * dx_hat * x)
//   acc += dx_hat * x * r              (this lane's dims of the dw partial)
// dy' (bf16) sits in the wave's LDS rows `dyl` (256 bytes each, 16-byte
// chunks at logical ^ swz(row)); a row's rotary angles pass through `ang`
// (4 rows x 64 floats), where lane t of the row computes angles t and t + 16.
// Rows at or past nrows read row nrows - 1 and store nothing.  Only this
// wave touches `dyl` and `ang`.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void row_bwd_wave(const lds_u8* dyl, lds_u8* ang, const uint16_t* x,
                                             uint16_t* dx, long long rstride, int nrows,
                                             long long pos0, const float* __restrict__ w,
                                             int rope_half, float eps, const RopeTable& tab,
                                             float acc[8]) {
  const int lane = threadIdx.x & 63, slot = lane >> 4, c16 = lane & 15;
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
  const int R = 2 * rope_half;
  static_assert(kMaxRopeHalf <= 32, "two angles per lane");
  const uint64_t fr0 = c16 < rope_half ? tab.frac[c16] : 0;
  const uint64_t fr1 = c16 + 16 < rope_half ? tab.frac[c16 + 16] : 0;
  u32x4 xu[8];
#pragma unroll
  for (int n = 0; n < 8; ++n)
    xu[n] = ld16(x + (long long)min(4 * n + slot, nrows - 1) * rstride + 8 * c16);
  lds_f32* cs = reinterpret_cast<lds_f32*>(ang) + 64 * slot;
  lds_f32* sn = cs + 32;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = 4 * n + slot;
    const lds_u8* rp = dyl + row * kRowB;
    float xv[8], dyv[8];
    unpack_bf16x8(xu[n], xv);
    unpack_bf16x8(__builtin_bit_cast(u32x4, lds_read_b128(rp + ((c16 ^ swz(row)) << 4))), dyv);
    float dh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dh[e] = dyv[e];
    if (R > 0) {
      const long long pos = pos0 + row;
      float c0, s0, c1, s1;
      if (c16 < rope_half) {
        rope_cos_sin_f(fr0, pos, c0, s0);
        cs[c16] = c0;
        sn[c16] = s0;
      }
      if (c16 + 16 < rope_half) {
        rope_cos_sin_f(fr1, pos, c1, s1);
        cs[c16 + 16] = c1;
        sn[c16 + 16] = s1;
      }
      wave_lds_sync();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * c16 + e;
        if (d < R) {
          const int t = d < rope_half ? d : d - rope_half;
          const int dp = d < rope_half ? d + rope_half : d - rope_half;  // rotary partner
          const float pv = __uint_as_float(
              (uint32_t)*reinterpret_cast<const lds_u16*>(rp + (((uint32_t)(dp >> 3) ^ swz(row)) << 4) +
                                                          2 * (dp & 7))
              << 16);
          const float c = cs[t], sg = sn[t];
          if (d < rope_half) dh[e] = dyv[e] * c + pv * sg;
          else dh[e] = dyv[e] * c - pv * sg;
        }
      }
      wave_lds_sync();  // the next pass rewrites the angles
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
    if (row < nrows) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = r * wl[e] * dh[e] - xv[e] * k3;
        acc[e] += dh[e] * xv[e] * r;
      }
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
      st16(dx + (long long)row * rstride + 8 * c16, u);
    }
  }
}

// Epilogue shared by the dq' and dk'/dv kernels, after their last barrier
// (every tile read, no copy in flight, so all of the LDS is free): the
// wave's 32 x 128 gradient accumulators (register r of block bd = dim
// 32 bd + 8 (r/4) + 4 half + r%4 of row l%32), times `scale` and rounded to
// bf16, go to its LDS rows; row_bwd_wave takes them to dx; the workgroup's
// partial sum of dw goes to row part_row of part (numbered by the rows the
// workgroup covers, not by launch order, so that the sum's order does not
// depend on the schedule).  LDS: 8 KB of rows and 1 KB of
// angles per wave, then 4 x 512 bytes for the partials (38 KB in all).
constexpr int kEpiRows = 0, kEpiAng = 4 * kTileB, kEpiRed = kEpiAng + 4 * 1024;
constexpr int kEpiBytes = kEpiRed + 4 * kD * 4;

__device__ __forceinline__ void grad_rows_epilogue(lds_u8* smem, const f32x16 (&a)[4], float scale,
                                                   const uint16_t* x, uint16_t* dx,
                                                   long long rstride, int nrows, long long pos0,
                                                   const float* __restrict__ w, int rope_half,
                                                   float eps, const RopeTable& tab,
                                                   float* __restrict__ part, long long part_row) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qcol = lane & 31, half = lane >> 5;
  lds_u8* rows = smem + kEpiRows + wvu * kTileB;
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 v;
      v[0] = pack_bf16x2(a[bd][4 * q4] * scale, a[bd][4 * q4 + 1] * scale);
      v[1] = pack_bf16x2(a[bd][4 * q4 + 2] * scale, a[bd][4 * q4 + 3] * scale);
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          rows + qcol * kRowB + (((uint32_t)(4 * bd + q4) ^ swz(qcol)) << 4) + 8 * half) = v;
    }
  wave_lds_sync();
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (nrows > 0)
    row_bwd_wave(rows, smem + kEpiAng + wvu * 1024, x, dx, rstride, nrows, pos0, w, rope_half, eps,
                 tab, acc);
  // the wave's four row slots, then the four waves in order
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  lds_f32* red = reinterpret_cast<lds_f32*>(smem + kEpiRed);
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wvu * kD + 8 * lane + e] = acc[e];
  }
  lds_barrier();
  if (tid < kD)
    part[part_row * kD + tid] =
        ((red[tid] + red[kD + tid]) + red[2 * kD + tid]) + red[3 * kD + tid];
}

// ---------------------------------------------------------------------------
// Per query row (b, s, h): Dr = sum dY*Y, dO = dY*sig(G), dG = dY*Y*(1-sig(G)),
// nlse2 = -LSE*log2(e) (the seed of the score products, whose result is
// then the exp2 argument of P itself).  Rows are enumerated over
// (b, h, s < Spad); rows past S get nlse2 = -inf and Dr = 0, so that they
// contribute P = 0 downstream.
// 16 lanes per row, 8 dims each.
// The same launch recomputes K' (the first kp.blocks blocks, 16 key rows
// each, with the key prologue's row code and so its bits): both passes are
// bound by HBM, and the small K' pass alone would run well below it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ dy,
                                                       const uint16_t* __restrict__ y,
                                                       const uint16_t* __restrict__ gate,
                                                       const float* __restrict__ lse,
                                                       uint16_t* __restrict__ dO,
                                                       uint16_t* __restrict__ dgate,
                                                       float* __restrict__ nlse2,
                                                       float* __restrict__ dvec, int B, int S,
                                                       int Spad, int Hq, KPrimeJob kp) {
  if ((long long)blockIdx.x < kp.blocks) {
    // K' of key rows 16 b .. 16 b + 15 (rows are (batch, position, kv head))
    __shared__ float xs[16][kD];
    __shared__ float cs[16][kMaxRopeHalf], sn[16][kMaxRopeHalf];
    const int lrow = threadIdx.x / 16, c16 = threadIdx.x % 16;
    const long long row = (long long)blockIdx.x * 16 + lrow;
    float x[8];
    unpack_bf16x8(ld16(kp.k + min(row, kp.rows - 1) * kD + 8 * c16), x);
    const RowConsts kc = row_consts(kp.w, kp.rope_half, kp.tab, c16);
    const long long s = (row / kp.Hkv) % kp.S;
    const int ref = lrow - (int)min(row % kp.Hkv, (long long)lrow);
    norm_rope_row(x, c16, kc, kp.eps, kp.rope_half, kp.pos_offset + s, xs[lrow], ref == lrow,
                  cs[lrow], sn[lrow], cs[ref], sn[ref]);
    if (row < kp.rows) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      st16(kp.kout + row * kD + 8 * c16, o);
    }
    return;
  }
  const long long row = ((long long)blockIdx.x - kp.blocks) * 16 + (threadIdx.x >> 4);
  const int c16 = threadIdx.x & 15;
  if (row >= (long long)B * Hq * Spad) return;  // whole 16-lane groups leave together
  const int s = (int)(row % Spad);
  const long long bh = row / Spad;
  if (s >= S) {
    if (c16 == 0) {
      nlse2[row] = -INFINITY;
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
    nlse2[row] = -(lse[bh * S + s] * kLog2e);
    dvec[row] = d;
  }
}

// ---------------------------------------------------------------------------
// dq': one 256-thread workgroup = (batch, kv head g, block of query
// positions), its 4 waves the group's query heads (as in the forward).  Per
// 32-key tile and wave:
//   S^T  = K' Q'^T   (A = K' rows, ds_read_b128; B = Q' in registers)
//   dP^T = V dO^T    (A = V rows, ds_read_b128; B = dO in registers)
//   P^T = exp2(S^T c - lse2), dS^T = P^T (dP^T - Dr), with S^T c - lse2 the
//   score product itself: its B operand is Q' c (rounded to bf16 as the
//   forward rounds it) and its accumulator starts at -lse2
//   dQ^T += K'^T dS^T (A = K'^T by transposing reads; B = dS^T as bf16)
// K'/V tiles come through a three-stage ring of untracked copies.
// ---------------------------------------------------------------------------
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
  // ---- this lane's query row: Q' c and dO as B operands, -lse2 and Dr
  const long long qrow = ((long long)b * p.S + (qok ? qi : 0)) * p.Hq + head;
  const long long lrw = ((long long)b * p.Hq + head) * p.Spad + qi;  // qi < Spad
  const float nl_l = p.nlse2[lrw];
  const float d_l = p.dvec[lrw];
  // The loop reads the registers loaded here; pin_row() has their loads land
  // before it (and before the tile copies that follow them are issued).
  // Otherwise the compiler, which does not see the tile copies, waits for
  // its loads inside the loop with a vmcnt that also drains the copies just
  // issued.
  bf16x8 qf[8], of[8];
  auto pin_row = [&]() __attribute__((always_inline)) {
    pin(nl_l);
    pin(d_l);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      pin(qf[kk]);
      pin(of[kk]);
    }
  };
  if constexpr (RH >= 0) {
    // Start-up as in the forward: tile 0 and the wave's 32 query rows are
    // requested together, the rows straight into LDS (16 lanes per 256-byte
    // row, in the stages tiles 1 and 2 will use: K' stages 1, 2 for waves 0,
    // 1, V stages 1, 2 for waves 2, 3), the dO half rows into registers.
    // Q' goes back out through the same LDS rows, row-coalesced; tile 1 is
    // requested once every wave is done with them.
    gload(t_hi, 0);
    lds_u8* qrows = smem + (wvu < 2 ? (1 + wvu) * kTileB : kVOff + (wvu - 1) * kTileB);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int row = 4 * n + (lane >> 4);
      const long long qr = ((long long)b * p.S + min(wrow0 + row, p.S - 1)) * p.Hq + head;
      dma16(p.q + qr * kD + 8 * ((uint32_t)(lane & 15) ^ swz(row)), lds_addr(qrows + n * 1024));
    }
    {
      const uint16_t* os = p.dO + qrow * kD + 64 * half;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        of[j] = __builtin_bit_cast(bf16x8, qok ? ld16(os + 8 * j) : u32x4{0, 0, 0, 0});
    }
    // Q' of this lane's half row: RMSNorm (+ weight) and the rotary pairs
    // (t, t + RH), with the same expressions in the same order as the
    // forward's fused query prologue, so that these are the bits the forward
    // multiplied.  Written to p.qp for the dk'/dv kernel.
    wait_vm<8>();  // the query rows (the dO loads after them may fly)
    const lds_u8* qr = qrows + qcol * kRowB;
    float x[64];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 v = lds_read_b128(qr + (((uint32_t)(8 * half + j) ^ swz(qcol)) << 4));
      unpack_bf16x8(__builtin_bit_cast(u32x4, v), x + 8 * j);
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
    // the score operand: Q' times c, rounded as the forward rounds it
#pragma unroll
    for (int d = 0; d < 64; ++d) x[d] *= p.scale_log2;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = pack_bf16x8(x + 8 * kk);
    // Q' c over the query half rows in LDS (each lane rewrites what it
    // read), then out row-coalesced for the dk'/dv kernel: lane L stores the
    // chunk it would have copied
    lds_u8* qw = qrows + qcol * kRowB;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(
          qw + (((uint32_t)(8 * half + j) ^ swz(qcol)) << 4)) = qf[j];
    wave_lds_sync();
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int row = 4 * n + (lane >> 4);
      if (wrow0 + row < p.S) {
        const u32x4 v = __builtin_bit_cast(
            u32x4, lds_read_b128(qrows + row * kRowB + ((uint32_t)(lane & 15) << 4)));
        uint16_t* dst = const_cast<uint16_t*>(p.qp) +
                        (((long long)b * p.S + wrow0 + row) * p.Hq + head) * kD +
                        8 * ((uint32_t)(lane & 15) ^ swz(row));
        st16(dst, v);
      }
    }
    pin_row();
    // every wave is done with its query rows: tile 1 may take their stage
    lds_barrier();
    if (nt > 1) gload(t_hi - 1, 1);
  } else {
    const uint16_t* os = p.dO + qrow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      of[j] = __builtin_bit_cast(bf16x8, qok ? ld16(os + 8 * j) : u32x4{0, 0, 0, 0});
    // the score operand Q' * c, formed by the key prologue
    const uint16_t* qs = p.qp + qrow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qf[j] = __builtin_bit_cast(bf16x8, qok ? ld16(qs + 8 * j) : u32x4{0, 0, 0, 0});
    pin_row();
    gload(t_hi, 0);
    if (nt > 1) gload(t_hi - 1, 1);
  }

  const uint32_t bread = (uint32_t)qcol * kRowB + (((uint32_t)(8 * half) ^ swz(qcol)) << 4);
  const TrOffsets tro = tr_offsets(lane);

  f32x16 acc[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) acc[bd] = f32x16{};

  if (nt > 1) sync_tiles<4>();
  else sync_tiles<0>();

  // Tile j in stage j % 3; the stage is a compile-time constant (the loop
  // below runs tiles in threes), so that every LDS address in the step is a
  // per-lane base plus an immediate.
  auto step = [&](int j, auto stg_tag) __attribute__((always_inline)) {
    constexpr int stg = decltype(stg_tag)::value;
    const int t = t_hi - j;
    const bool issue = j + 2 < nt;
    if (issue) gload(t - 2, stg == 0 ? 2 : stg - 1);
    const lds_u8* kt = smem + stg * kTileB;
    const lds_u8* vt = kt + kVOff;
    // With fewer than four heads per workgroup its waves hold different
    // query rows; a wave that sees none of the tile's keys (its rows lie
    // wholly before the tile or a band past it) has only zero products
    // to add and skips them.
    const bool active = t * 32 <= wrow0 + 31 && wrow0 - (t * 32 + 31) < lim;
    if (active) {
      f32x16 sT, dpT = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[r] = nl_l;  // every register is this lane's query
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kt + (bread ^ (uint32_t)(kk << 4))),
                                                     qf[kk], sT, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        dpT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(vt + (bread ^ (uint32_t)(kk << 4))),
                                                      of[kk], dpT, 0, 0, 0);
      // register r: key t*32 + 8(r/4) + 4 half + r%4 of this lane's query.
      // Only a tile that reaches past the wave's first query or below its
      // last query's band needs the mask (a wave-uniform branch).
      const bool masked = t * 32 + 31 > wrow0 || wrow0 + 31 - t * 32 >= lim;
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(sT[r]);
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dq = qi - (t * 32 + 8 * (r >> 2) + 4 * half + (r & 3));
          ds[r] = (unsigned)dq < (unsigned)lim ? ds[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = ds[r] * (dpT[r] - d_l);  // P (dP - Dr)
      const bf16x8 dsf0 = pack_bf16x8(ds), dsf1 = pack_bf16x8(ds + 8);
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
        acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kt, tro, bd, 0), dsf0, acc[bd], 0, 0, 0);
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
        acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kt, tro, bd, 1), dsf1, acc[bd], 0, 0, 0);
      // each score / dP MFMA after its LDS operand read (left to the
      // scheduler, the reads went first in a block: 1-2% slower)
#pragma unroll
      for (int gg = 0; gg < 16; ++gg) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
    }
    // tile j+1 must have landed; tile j+2's four copies may still fly
    if (issue) sync_tiles<4>();
    else sync_tiles<0>();
  };
  for (int j = 0; j < nt; j += 3) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < nt) step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < nt) step(j + 2, std::integral_constant<int, 2>{});
  }

  // dq' = tau * dQ, then back through RoPE and RMSNorm to dq
  static_assert(kEpiBytes <= 2 * NS * kTileB, "the epilogue fits the tile ring");
  grad_rows_epilogue(smem, acc, p.scale, p.q + (((long long)b * p.S + wrow0) * p.Hq + head) * kD,
                     p.dq + (((long long)b * p.S + wrow0) * p.Hq + head) * kD,
                     (long long)p.Hq * kD, min(32, p.S - wrow0), p.pos_offset + wrow0, p.q_norm_w,
                     p.rope_half, p.eps, p.tab, p.part_q, (long long)pb * geo.n_bhg + bhg);
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
//   P = exp2(S c - lse2), dS = P (dP - Dr), with S c - lse2 the score
//   product itself: A = Q' c (the dq' kernel writes it, rounded as the
//   forward rounds it), its accumulator starting at -lse2 of the tile's rows;
//   dK then accumulates (Q' c)^T dS and takes tau / c at the end
//   dV^T += dO^T P, dK^T += Q'^T dS  (A by transposing reads; B = P, dS)
// The block's V rows sit in LDS for the whole kernel (keeping them in
// registers would leave room for one wave per SIMD only); Q'/dO tiles and
// the tile's lse2 / Dr come through a two-stage ring of untracked copies
// (five per wave and tile).
// ---------------------------------------------------------------------------
constexpr int kDkvStage = 2 * kTileB + 256;  // Q', dO, nlse2[32], Dr[32]
constexpr int kDkvV = 2 * kDkvStage;         // V rows of the key block, 4 x 8 KB

// BANDED: 0 < window < S.  A global layer (window 0, or at least S) masks
// only the visits at the diagonal, under a wave-uniform branch; a band masks
// every element (most of its visits cross an edge of the band).
template <bool BANDED>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * kDkvStage + 4 * kTileB];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int qcol = lane & 31, half = lane >> 5;
  const int grp = p.Hq / p.Hkv;
  const bool banded = BANDED;
  const int lim = BANDED ? p.window : 0x7fffffff;

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

  // ---- copies: Q' / dO rows 4(2w+j) + L/16 of the tile; nlse2 / Dr: lanes
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
      // rows past S read row S-1 (their nlse2 is -inf, so P = 0)
      const uint32_t off = (uint32_t)((min(q0 + lrow[j], p.S - 1) - q0) * qstride * 2) + chk[j];
      dma16_s(qb, off, sb + (2 * wvu + j) * 1024);
      dma16_s(ob, off, sb + kTileB + (2 * wvu + j) * 1024);
    }
    const long long vrow = ((long long)b * p.Hq + head) * p.Spad + q0;
    if (lane < 4) {
      const float* src = (wvu < 2 ? p.nlse2 : p.dvec) + vrow + 16 * (wvu & 1) + 4 * lane;
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
  // the K' loads land here, not inside the loop (see the dq' kernel)
#pragma unroll
  for (int j = 0; j < 8; ++j) pin(kf[j]);
  const lds_u8* vblk = smem + kDkvV + wvu * kTileB;  // this wave's V rows
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

  const int kw = kb0 + 32 * wvu;  // the wave's first key
  // Visit i in stage stg; the stage is a compile-time constant (the loop
  // below runs visits in pairs), so that every LDS address in the visit is a
  // per-lane base plus an immediate.
  auto visit = [&](int i, auto stg_tag) __attribute__((always_inline)) {
    constexpr int stg = decltype(stg_tag)::value;
    const int q0 = (qt_lo + nq - 1 - i / grp) * 32;
    const lds_u8* qt = smem + stg * kDkvStage;
    const lds_u8* ot = qt + kTileB;
    const lds_u8* lt = qt + 2 * kTileB;
    // A wave whose 32 keys see none of the tile's 32 queries (on a band, a
    // third of the visits: the block's visits span its 128 keys' band) has
    // only zero products to add; it skips them and leaves its SIMD to the
    // other workgroup, but still takes part in the copies and barriers.
    const bool active = q0 + 31 >= kw && q0 - (kw + 31) < lim;
    if (active) {
      // the score accumulator starts at -lse2 of its query (register r:
      // query q0 + 8(r/4) + 4 half + r%4)
      f32x16 s, dp = f32x16{};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 l4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
            lt + 4 * (8 * m + 4 * half));
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * m + e] = l4[e];
      }
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
        const f32x4 d4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
            lt + 128 + 4 * (8 * m + 4 * half));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          float x = fast_exp2(s[r]);
          if constexpr (BANDED) {
            const int dq = q0 + 8 * m + 4 * half + e - kj;
            x = (unsigned)dq < (unsigned)lim ? x : 0.f;
          }
          pr[r] = x;
          ds[r] = x * (dp[r] - d4[e]);
        }
      }
      if constexpr (!BANDED) {
        // causal: only a visit whose queries reach below the wave's last key
        if (q0 < kw + 31) {
          const int dq0 = q0 + 4 * half - kj;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = dq0 + 8 * (r >> 2) + (r & 3) >= 0;
            pr[r] = ok ? pr[r] : 0.f;
            ds[r] = ok ? ds[r] : 0.f;
          }
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
      // each score MFMA after its operand read and each dP MFMA after its
      // two (left to the scheduler, the reads went first: 1-2% slower)
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
    }
    // tile i+1 has landed and every wave is done with tile i; then tile i+2
    // goes into tile i's stage
    sync_tiles<0>();
    if (i + 2 < ntile) gload(i + 2, stg);
  };
  for (int i = 0; i < ntile; i += 2) {
    visit(i, std::integral_constant<int, 0>{});
    if (i + 1 < ntile) visit(i + 1, std::integral_constant<int, 1>{});
  }

  // register r of block bd -> dim 32bd + 8(r/4) + 4 half + r%4 of key kj
  if (kok) {
    const long long krow = ((long long)b * p.S + kj) * p.Hkv + g;
    uint16_t* dvd = p.dv + krow * kD + 4 * half;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 w;
        w.x = pack_bf16x2(dvv[bd][4 * q4], dvv[bd][4 * q4 + 1]);
        w.y = pack_bf16x2(dvv[bd][4 * q4 + 2], dvv[bd][4 * q4 + 3]);
        *reinterpret_cast<uint2*>(dvd + 32 * bd + 8 * q4) = w;
      }
  }
  // dk' = tau * dK = (tau / c) * (Q' c)^T dS, then back through RoPE and
  // RMSNorm to dk
  static_assert(kEpiBytes <= 2 * kDkvStage + 4 * kTileB, "the epilogue fits the LDS");
  const int r0 = kb0 + 32 * wvu;
  grad_rows_epilogue(smem, dk, p.scale / p.scale_log2, p.k + (((long long)b * p.S + r0) * p.Hkv + g) * kD,
                     p.dk + (((long long)b * p.S + r0) * p.Hkv + g) * kD, (long long)p.Hkv * kD,
                     min(32, p.S - r0), p.pos_offset + r0, p.k_norm_w, p.rope_half, p.eps, p.tab,
                     p.part_k, bid);
}

// ---------------------------------------------------------------------------
// Norm-weight gradients: dw = the sum of one gradient's n partials (the
// workgroups of the dq' kernel for q, of the dk'/dv kernel for k) in a fixed
// order, so that every run gives the same bits.  reduce_chunks_kernel:
// block (j, which) sums rows j*ch .. j*ch + ch - 1 in order
// (ch = ceil(n / kBwdRedChunks)); reduce_final_kernel adds the chunk sums of
// gradient `which` in order (eight runs of 32, then the eight in order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kD) void reduce_chunks_kernel(const float* __restrict__ part_q,
                                                           long long nq,
                                                           const float* __restrict__ part_k,
                                                           long long nk, float* __restrict__ red) {
  const int which = blockIdx.y, j = blockIdx.x, d = threadIdx.x;
  const float* part = which ? part_k : part_q;
  const long long n = which ? nk : nq;
  const long long ch = (n + kBwdRedChunks - 1) / kBwdRedChunks;
  const long long r0 = j * ch, r1 = min(n, r0 + ch);
  float s = 0.f;
  for (long long r = r0; r < r1; ++r) s += part[r * kD + d];
  red[((long long)which * kBwdRedChunks + j) * kD + d] = s;
}

constexpr int kRedRuns = 8;
static_assert(kBwdRedChunks % kRedRuns == 0, "chunk sums split evenly over the runs");
__global__ __launch_bounds__(kRedRuns * kD) void reduce_final_kernel(const float* __restrict__ red,
                                                                     float* __restrict__ dwq,
                                                                     float* __restrict__ dwk) {
  constexpr int kRun = kBwdRedChunks / kRedRuns;
  __shared__ float runs[kRedRuns][kD];
  const int which = blockIdx.x;
  const int d = threadIdx.x % kD, c = threadIdx.x / kD;
  const float* src = red + ((long long)which * kBwdRedChunks + c * kRun) * kD + d;
  float s = 0.f;
#pragma unroll 8
  for (int k = 0; k < kRun; ++k) s += src[k * kD];
  runs[c][d] = s;
  __syncthreads();
  if (c == 0) {
    float t = runs[0][d];
#pragma unroll
    for (int j = 1; j < kRedRuns; ++j) t += runs[j][d];
    (which ? dwk : dwq)[d] = t;
  }
}

}  // namespace

hipError_t launch_bwd_prep(const uint16_t* dy, const uint16_t* y, const uint16_t* gate,
                           const float* lse, uint16_t* dO, uint16_t* dgate, float* nlse2,
                           float* dvec, int B, int S, int Spad, int Hq, KPrimeJob kp,
                           hipStream_t stream) {
  const long long rows = (long long)B * Hq * Spad;
  kp.blocks = (kp.rows + 15) / 16;
  const long long blocks = kp.blocks + (rows + 15) / 16;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dy, y, gate, lse,
                     dO, dgate, nlse2, dvec, B, S, Spad, Hq, kp);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const DqGeo geo = bwd_dq_geo(p.B, p.S, p.Hq, p.Hkv);
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
  const long long blocks = bwd_dkv_blocks(p.B, p.S, p.Hkv);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.window > 0 && p.window < p.S)
    hipLaunchKernelGGL(bwd_dkv_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_dkv_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(const BwdParams& p, float* red, float* dwq, float* dwk,
                               hipStream_t stream) {
  hipLaunchKernelGGL(reduce_chunks_kernel, dim3(kBwdRedChunks, 2), dim3(kD), 0, stream, p.part_q,
                     bwd_dq_blocks(p.B, p.S, p.Hq, p.Hkv), p.part_k,
                     bwd_dkv_blocks(p.B, p.S, p.Hkv), red);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_final_kernel, dim3(2), dim3(kRedRuns * kD), 0, stream, red, dwq, dwk);
  return hipGetLastError();
}

}  // namespace zg
