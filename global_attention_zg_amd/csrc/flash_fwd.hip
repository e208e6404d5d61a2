// Banded (sliding-window) and global causal flash attention, forward.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: a sliding-window layer
// lets each token attend only to its 128 neighbouring tokens; global layers
// attend over the whole causal prefix.  Section 核心方法: GQA, 32 query heads
// share 8 KV heads.  Page "7B 打 235B？…全开源配方" (shibing624.github.io),
// section 🏗️ 架构: the local attention output is multiplied by a sigmoid gate.
//
// One 256-thread workgroup = one KV head g and a block of query positions; its
// four waves are four query heads of g's group (GQA packing: every K/V tile
// in LDS feeds 4 x 32 query rows).  Each wave owns 32 query rows; lane l owns
// query row l%32 and the half l/32 of everything else, so the online softmax
// needs one cross-half exchange per tile and no other cross-lane traffic.
//
//   S^T = K' Q'^T  (v_mfma_f32_32x32x16_bf16, A = K' tile rows from LDS,
//                   B = the wave's normalised + rotated Q' in registers)
//   O^T += V^T P^T (A = V^T tile from LDS, B = P in registers)
//
// Only KV tiles that intersect the causal band of the workgroup's queries are
// visited: for a window W that is ceil((32 + W - 1) / 64) tiles, for the
// global layer every tile up to the diagonal.  The query prologue (RMSNorm +
// partial RoPE) is fused into the Q load; the sigmoid gate is fused into the
// epilogue.  Softmax runs in fp32 on raw scores with exp2(fma(s, c, -m c)),
// c = scale*log2(e), and lazy rescaling of the accumulator (only when the
// running max grows by more than 2^8 in exp2 units).

#include "zg_common.h"
#include "zg_launch.h"

namespace zg {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;             // keys per KV tile
constexpr int kKsStride = kD + 8;   // bf16 per K' row in LDS (272 B: 16-B aligned, skewed banks)
constexpr int kVtStride = kBN + 8;  // bf16 per V^T row in LDS (144 B)
constexpr int kKsElems = kBN * kKsStride;
constexpr int kVtElems = kD * kVtStride;
constexpr int kBufElems = kKsElems + kVtElems;  // one K'+V^T stage: 35840 B
constexpr float kRescaleThreshold = 8.0f;       // log2 units

struct Geo {
  int heads_per_wg;  // query heads per workgroup (= waves sharing positions)
  int pos_per_wg;    // query positions per workgroup
  int n_pos_blocks;
  int hgroups;       // workgroups per (b, kv head, position block)
  int n_bhg;         // B * Hkv * hgroups
};

// Row of the 32-key block that MFMA row m reads: swaps bits 2 and 3 of m so
// that output registers 8t..8t+7 of lane half h hold keys 16t+8h .. 16t+8h+7,
// i.e. exactly the B operand of the P.V product for k-step t.
__device__ __forceinline__ int key_row_of(int m) {
  return (m & 16) | ((m & 4) << 1) | ((m & 8) >> 1) | (m & 3);
}
// Row of V^T (a head dim) that MFMA row m of output block bd reads: chosen so
// that output register r of lane half h holds dim 64h + 16bd + r.
__device__ __forceinline__ int dim_row_of(int bd, int m) {
  return ((m >> 2) & 1) * 64 + bd * 16 + (m >> 3) * 4 + (m & 3);
}

__global__ __launch_bounds__(kThreads, 2) void flash_fwd_kernel(FlashParams p, Geo geo) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBufElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int qcol = lane & 31;
  const int half = lane >> 5;
  const int grp = p.Hq / p.Hkv;

  // ---- workgroup -> (position block, batch, kv head, head group)
  const int bid = blockIdx.x;
  const int bhg = bid % geo.n_bhg;
  int pb = bid / geo.n_bhg;
  if (p.window == 0) pb = geo.n_pos_blocks - 1 - pb;  // longest causal rows first
  const int hg = bhg % geo.hgroups;
  const int bgi = bhg / geo.hgroups;
  const int g = bgi % p.Hkv;
  const int b = bgi / p.Hkv;
  const int head = g * grp + hg * geo.heads_per_wg + (wv % geo.heads_per_wg);
  const int i0w = pb * geo.pos_per_wg;
  const int qi = i0w + (wv / geo.heads_per_wg) * 32 + qcol;
  const bool qok = qi < p.S;
  const int hi = min(p.S, i0w + geo.pos_per_wg);
  const int lo = p.window > 0 ? max(0, i0w - p.window + 1) : 0;
  const int nt = (hi - lo + kBN - 1) / kBN;
  const int kfirst = hi - nt * kBN;  // tiles end exactly at the last query; may start < 0

  // ---- fused query prologue: RMSNorm (+ weight), partial RoPE, -> bf16 B operand
  const long long qrow = ((long long)b * p.S + (qok ? qi : 0)) * p.Hq + head;
  bf16x8 qf[8];
  {
    float x[64];
    const uint16_t* src = p.q + qrow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 u = qok ? ld16(src + 8 * j) : u32x4{0, 0, 0, 0};
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
      u32x4 wv4 = ld16(wsrc + 4 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * j + i] *= r * __uint_as_float(wv4[i]);
    }
    if (p.rope_half > 0 && half == 0) {
      // rotary dims (all < 64) live in the lane-half-0 registers; go through a
      // private LDS row so the partner dim can be addressed at run time.
      float* qs = reinterpret_cast<float*>(smem) + (wv * 32 + qcol) * 65;
#pragma unroll
      for (int d = 0; d < 64; ++d) qs[d] = x[d];
      const long long pos = p.pos_offset + qi;
      const int rh = p.rope_half;
#pragma unroll
      for (int t = 0; t < kMaxRopeHalf; ++t) {
        if (t < rh) {
          float c, s;
          rope_cos_sin(p.tab, t, pos, c, s);
          const float a = qs[t], bb = qs[t + rh];
          qs[t] = a * c - bb * s;
          qs[t + rh] = bb * c + a * s;
        }
      }
#pragma unroll
      for (int d = 0; d < 64; ++d) x[d] = qs[d];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = pack_bf16x8(x + 8 * kk);
  }
  __syncthreads();  // the prologue's LDS rows are reused by the KV tiles

  // ---- KV tile staging: global -> registers -> LDS (K' row-major, V transposed)
  const long long kvstride = (long long)p.Hkv * kD;
  const uint16_t* kbase = p.kp + (long long)b * p.S * kvstride + g * kD;
  const uint16_t* vbase = p.v + (long long)b * p.S * kvstride + g * kD;
  const int lc = tid & 15;   // 16-byte column chunk
  const int lr = tid >> 4;   // 0..15
  u32x4 kreg[4], vreg[4];

  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kt + lr + 16 * j;
      kreg[j] = key >= 0 ? ld16(kbase + key * kvstride + 8 * lc) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kt + 4 * lr + j;
      vreg[j] = key >= 0 ? ld16(vbase + key * kvstride + 8 * lc) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* Ks = smem + buf * kBufElems;
    uint16_t* Vt = Ks + kKsElems;
#pragma unroll
    for (int j = 0; j < 4; ++j) st16(Ks + (lr + 16 * j) * kKsStride + 8 * lc, kreg[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int wd = i >> 1;
      uint32_t a, c;
      if (i & 1) {
        a = (vreg[0][wd] >> 16) | (vreg[1][wd] & 0xffff0000u);
        c = (vreg[2][wd] >> 16) | (vreg[3][wd] & 0xffff0000u);
      } else {
        a = (vreg[0][wd] & 0xffffu) | (vreg[1][wd] << 16);
        c = (vreg[2][wd] & 0xffffu) | (vreg[3][wd] << 16);
      }
      uint2 pr = {a, c};
      *reinterpret_cast<uint2*>(Vt + (8 * lc + i) * kVtStride + 4 * lr) = pr;
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) acc[bd] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const int mrow = lane & 31;
  const int krow = key_row_of(mrow);
  const float rescale_raw = kRescaleThreshold / p.scale_log2;  // threshold in raw score units

  gload(kfirst);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int kt = kfirst + t * kBN;
    if (t + 1 < nt) gload(kt + kBN);
    const uint16_t* Ks = smem + (t & 1) * kBufElems;
    const uint16_t* Vt = Ks + kKsElems;

    // S^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x16{};
      const uint16_t* kr = Ks + (blk * 32 + krow) * kKsStride + 64 * half;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 8 * kk);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[blk], 0, 0, 0);
      }
    }

    // mask (raw scores), running max in raw units; exp2 argument is one FMA
    // fma(s, c, -m*c) so that masked and unmasked tiles round identically
    const bool need_mask = p.window > 0 || kt < 0 || kt + kBN - 1 > i0w;
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[blk][r];
        if (need_mask) {
          const int j = kt + blk * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
          const bool vis = j >= 0 && j <= qi && (p.window == 0 || qi - j < p.window);
          v = vis ? v : -INFINITY;
        }
        s[blk][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = pair_max32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + rescale_raw)) {
      const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2((m_run - m_new) * p.scale_log2);
#pragma unroll
      for (int bd = 0; bd < 4; ++bd) acc[bd] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg_mc = m_run == -INFINITY ? 0.0f : -m_run * p.scale_log2;

    bf16x8 pf[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = fast_exp2(__builtin_fmaf(s[blk][r], p.scale_log2, neg_mc));
        l_run += pv[r];
      }
      pf[blk][0] = pack_bf16x8(pv);
      pf[blk][1] = pack_bf16x8(pv + 8);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int bd = 0; bd < 4; ++bd) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              Vt + dim_row_of(bd, mrow) * kVtStride + blk * 32 + 16 * tt + 8 * half);
          acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[blk][tt], acc[bd], 0, 0, 0);
        }
      }
    }

    if (t + 1 < nt) sstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, store
  const float l_tot = pair_sum32(l_run);
  const float inv = 1.0f / l_tot;
  if (qok) {
    uint16_t* dst = p.out + qrow * kD + 64 * half;
    const uint16_t* gsrc = p.gate ? p.gate + qrow * kD + 64 * half : nullptr;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      float o[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = acc[bd][r] * inv;
      if (gsrc) {
        float gv[16];
        unpack_bf16x8(ld16(gsrc + 16 * bd), gv);
        unpack_bf16x8(ld16(gsrc + 16 * bd + 8), gv + 8);
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] *= sigmoidf_(gv[r]);
      }
      u32x4 w0, w1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
        w1[i] = pack_bf16x2(o[8 + 2 * i], o[8 + 2 * i + 1]);
      }
      st16(dst + 16 * bd, w0);
      st16(dst + 16 * bd + 8, w1);
    }
    if (p.lse && half == 0)
      p.lse[((long long)b * p.Hq + head) * p.S + qi] =
          (m_run * p.scale_log2 + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_flash_fwd(const FlashParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const int grp = p.Hq / p.Hkv;
  Geo geo;
  geo.heads_per_wg = grp < kWaves ? grp : kWaves;
  geo.hgroups = grp / geo.heads_per_wg;
  geo.pos_per_wg = 32 * kWaves / geo.heads_per_wg;
  geo.n_pos_blocks = (p.S + geo.pos_per_wg - 1) / geo.pos_per_wg;
  geo.n_bhg = p.B * p.Hkv * geo.hgroups;
  const long long blocks = (long long)geo.n_pos_blocks * geo.n_bhg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(flash_fwd_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p,
                     geo);
  return hipGetLastError();
}

}  // namespace zg
