// Banded (sliding-window) and global causal flash attention, forward.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: a sliding-window layer
// lets each token attend only to its 128 neighbouring tokens; global layers
// attend over the whole causal prefix.  Section 核心方法: GQA, 32 query heads
// share 8 KV heads.  Page "7B 打 235B？…全开源配方" (shibing624.github.io),
// section 🏗️ 架构: the local attention output is multiplied by a sigmoid gate.
//
// A workgroup serves one KV head g and a block of query positions; each wave
// is one query head of g's group at 32 positions (GQA packing: every K'/V
// tile in LDS feeds all of the workgroup's waves).  Windowed layers use four
// waves (the four heads at 32 positions), global layers eight (the four
// heads at 64 positions).  Lane l owns query row l%32 and the half l/32 of
// everything else, so the online softmax needs one cross-half exchange per
// tile and no other cross-lane traffic.
//
//   S^T = K' Q'^T  (v_mfma_f32_32x32x16_bf16, A = K' tile rows from LDS,
//                   B = the wave's normalised + rotated Q' in registers)
//   O^T += V^T P^T (A = V^T read from the row-major V tile with the gfx950
//                   transposing LDS load ds_read_b64_tr_b16, B = P in registers)
//
// K' and V tiles go from global memory straight into LDS (global_load_lds,
// no register staging) through a ring (three tile stages, or four pairs of
// tiles for the global layer), row-major with
// 256-byte rows whose 16-byte chunks are XOR-swizzled by row: chunk ^ (row &
// 15) for K', chunk ^ ((row & 3) << 2) for V.  With the 64-bank LDS every
// MFMA operand read is then free of bank conflicts, and each read address is
// a per-lane base plus an immediate.
//
// Only KV tiles that intersect the causal band of the workgroup's queries are
// visited: for a window W that is ceil((32 + W - 1) / 32) + 1 tiles at most,
// for the global layer every tile up to the diagonal.  The query prologue
// (RMSNorm + partial RoPE) is fused into the Q load; the sigmoid gate is
// fused into the epilogue.  Softmax runs in fp32 on raw scores with
// exp2(fma(s, c, -m c)), c = scale*log2(e), and lazy rescaling of the
// accumulator (only when the running max grows by more than 2^8 in exp2
// units).  In the global kernel the two waves that share a SIMD alternate
// between an MFMA phase and a softmax phase, so that one wave's softmax
// (VALU) runs under the other's matrix work; each phase covers a pair of
// tiles (64 keys), with one running-max update per pair.

#include <type_traits>

#include "zg_common.h"
#include "zg_launch.h"
#include "zg_lds.h"

namespace zg {

namespace {

// Windowed layers: 4 waves per workgroup (the four query heads of a KV group
// at 32 positions).  Global layers: 8 waves, the same four heads at 64
// positions, so that each K'/V tile copied into LDS feeds twice the work; the
// two waves that share a SIMD (w and w + 4) alternate MFMA and softmax phases.
template <bool BANDED> struct Cfg {
  static constexpr int kWaves = BANDED ? 4 : 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBlocksPerWave = 8 / kWaves;  // 1 KB blocks of each tile a wave copies
  static constexpr int kCopies = 2 * kBlocksPerWave;  // its K' + V copies per tile
};
constexpr int kBN = 32;                          // keys per KV tile (one MFMA block)
constexpr int kRowBytes = kD * 2;                // 256-byte K'/V rows in LDS, 16-byte chunks XOR-swizzled
constexpr int kTileBytes = kBN * kRowBytes;      // 8192 per K' or V stage
// LDS ring per K' and V, K' stages first, then the V stages.  Windowed
// layers: three tile stages, copies fly two tiles ahead.  Global layers work
// on pairs of tiles: four pair stages (eight tiles), copies fly two pairs
// ahead (the fourth stage holds the pair the other wave of the SIMD may
// still be reading).
template <bool BANDED> struct Ring {
  static constexpr int kStages = BANDED ? 3 : 8;
  static constexpr int kVOff = kStages * kTileBytes;
  static constexpr int kTilesBytes = 2 * kStages * kTileBytes;
};
constexpr int kQScratchBytes = Cfg<false>::kWaves * 32 * 65 * 4;  // query-prologue RoPE rows (reused)
constexpr int kSmemGlobal =
    Ring<false>::kTilesBytes > kQScratchBytes ? Ring<false>::kTilesBytes : kQScratchBytes;  // 131072
// Windowed layers also stage their query rows (8 KB per wave) behind the
// tiles, and after the loop their fp32 output rows (16 KB per wave) for
// coalesced stores.
constexpr int kQRegion = Ring<true>::kTilesBytes;
constexpr int kSmemBanded = Ring<true>::kTilesBytes + Cfg<true>::kWaves * 32 * kRowBytes;  // 81920
static_assert(Cfg<true>::kWaves * 32 * 128 * 4 <= kSmemBanded, "output staging must fit");
constexpr float kRescaleThreshold = 8.0f;        // exp2 units

struct Geo {
  int heads_per_wg;  // query heads per workgroup (= waves sharing positions)
  int pos_per_wg;    // query positions per workgroup
  int n_pos_blocks;
  int hgroups;       // workgroups per (b, kv head, position block)
  int n_bhg;         // B * Hkv * hgroups
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

__device__ __forceinline__ void pv_mfma(TileState& st, const bf16x8 (&va)[8], const bf16x8 (&pf)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
      st.acc[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[4 * t + bd], pf[t], st.acc[bd], 0, 0, 0);
  }
}

// BANDED: sliding-window layer (window > 0); otherwise global causal.
// RH: rope_dim / 2 when known at compile time (0 or 21: the rotation runs in
// registers), -1 for any other rope_dim (rotation through LDS).
template <bool BANDED, int RH, bool PACKED>
__global__ __launch_bounds__(Cfg<BANDED>::kThreads, 2) void flash_fwd_kernel(FlashParams p,
                                                                               Geo geo) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[BANDED ? kSmemBanded : kSmemGlobal];
  lds_u8* smem = (lds_u8*)smem_raw;  // generic -> LDS address space
  constexpr int NS = Ring<BANDED>::kStages;
  constexpr int kVOff = Ring<BANDED>::kVOff;

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
  if (!BANDED) pb = geo.n_pos_blocks - 1 - pb;  // longest causal rows first
  const int hg = bhg % geo.hgroups;
  const int bgi = bhg / geo.hgroups;
  const int g = bgi % p.Hkv;
  const int b = bgi / p.Hkv;
  const int head = g * grp + hg * geo.heads_per_wg + (wv % geo.heads_per_wg);
  const int i0w = pb * geo.pos_per_wg;
  // This workgroup's sequence is rows [tok0, tok0 + S) of the token-major
  // layout: tok0 = b * S for fixed-length batches; with cu_seqlens the
  // offsets are clamped into [0, total) and the length to the grid's S.
  int S = p.S;
  long long tok0 = (long long)b * p.S;
  long long lse0 = (long long)b * p.Hq * p.S, lse_hs = p.S;
  if constexpr (PACKED) {
    const long long c0 = min(max((long long)p.cu_seqlens[b], 0LL), p.total);
    const long long c1 = min(max((long long)p.cu_seqlens[b + 1], c0), p.total);
    tok0 = c0;
    S = (int)min(c1 - c0, (long long)p.S);
    lse0 = tok0;
    lse_hs = p.total;
    if (i0w >= S) return;  // whole workgroup: past the end of a short sequence
  }
  const int qi = i0w + (wv / geo.heads_per_wg) * 32 + qcol;
  const bool qok = qi < S;
  // Rows past the end are padding: give them row S-1's visibility so that the
  // wave-wide lazy-rescale vote is the same as for any window >= S.
  const int qm = min(qi, S - 1);
  const int lim = BANDED ? min(p.window, qm + 1) : qm + 1;
  const int hi = min(S, i0w + geo.pos_per_wg);      // keys < hi
  const int lo = BANDED ? max(0, i0w - p.window + 1) : 0;  // keys >= lo


  const long long qrow = (tok0 + (qok ? qi : 0)) * p.Hq + head;
  bf16x8 qf[8];  // this wave's Q' rows: the B operand of every S MFMA

  // ---- KV tile staging: global -> LDS directly (global_load_lds_dwordx4)
  // into a ring of NS stages, so that a tile's loads have NS - 1 tiles of
  // compute to arrive.  Wave wv fills the BPW 1 KB blocks BPW wv + j (rows
  // 4n..4n+3) of each 8 KB tile: lane L writes physical chunk L%16 of row
  // 4n + L/16 and so fetches the logical chunk that the row's swizzle places
  // there.
  constexpr int BPW = Cfg<BANDED>::kBlocksPerWave;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);  // wave-uniform copy
  const long long kvstride = (long long)p.Hkv * kD;
  const uint16_t* kbase = p.kp + tok0 * kvstride + g * kD;
  const uint16_t* vbase = p.v + tok0 * kvstride + g * kD;
  uint32_t row_off[2], kchunk[2];
  int lrow[2];
  const uint32_t vchunk = 16u * ((lane & 15) ^ (((lane >> 4) & 3) << 2));
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    lrow[j] = 4 * (BPW * wvu + j) + (lane >> 4);
    row_off[j] = (uint32_t)(lrow[j] * kvstride * 2);
    kchunk[j] = 16u * ((lane & 15) ^ (lrow[j] & 15));
  }
  // tile -> stage stg; keys >= S (only in the top tile) load key S-1 and are
  // masked out
  auto gload = [&](int t, int stg) {
    const unsigned char* kb = (const unsigned char*)(kbase + (long long)t * kBN * kvstride);
    const unsigned char* vb = (const unsigned char*)(vbase + (long long)t * kBN * kvstride);
    const uint32_t kl = lds_addr(smem + stg * kTileBytes + BPW * wvu * 1024);
    const uint32_t vl = kl + kVOff;
    if (t * kBN + kBN <= S) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        dma16_s(kb, row_off[j] + kchunk[j], kl + j * 1024);
        dma16_s(vb, row_off[j] + vchunk, vl + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const uint32_t off = (uint32_t)((min(t * kBN + lrow[j], S - 1) - t * kBN) * kvstride * 2);
        dma16_s(kb, off + kchunk[j], kl + j * 1024);
        dma16_s(vb, off + vchunk, vl + j * 1024);
      }
    }
  };

  TileState st;
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) st.acc[bd] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const float c = p.scale_log2;
  const float rescale_raw = kRescaleThreshold / c;  // threshold in raw score units
  // per-lane LDS read offsets: K' row q%32 at logical chunk 8h; V rows
  // 4h + i/4 at dims 32bd + 16 (group parity) + 4 (i%4) for the transposing loads
  const uint32_t kread_off = qcol * kRowBytes + ((uint32_t)((8 * half) ^ (qcol & 15)) << 4);
  const int gi = lane & 15;
  const int vq = gi >> 2;
  const int vlow = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
  const lds_u8* vread0[4];  // stage 0; stage k adds k * kTileBytes
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) {
    const int off = (4 * half + vq) * kRowBytes + (((bd ^ vq) << 2 | vlow) << 4) + 8 * (gi & 1);
    vread0[bd] = smem + kVOff + off;
  }

  // 32-key tiles aligned to key 0, visited from the diagonal down: tile
  // t = t_hi - j holds keys [32t, 32t + 32).  Masked tiles: every tile of a
  // windowed layer; for the global layer the tiles reaching past the
  // workgroup's first query.
  const int t_hi = (hi - 1) / kBN;
  const int nt = t_hi - lo / kBN + 1;
  // tile j lives in stage j % NS; loads for tile j + NS - 1 are issued while
  // tile j is computed, into the stage tile j - 1 used
  int stg = 0;
  auto step = [&](int j, auto mask_tag) {
    const int t = t_hi - j;
    const int stg_ahead = stg == 0 ? NS - 1 : stg - 1;  // (j + NS - 1) % NS
    const bool issue = j + NS - 1 < nt;
    if (issue) gload(t - (NS - 1), stg_ahead);
    f32x16 s;
    qk_blk(s, smem + stg * kTileBytes, kread_off, qf);
    if (decltype(mask_tag)::value) mask_blk(s, t * kBN, qm, lim, half);
    const float neg_mc = softmax_rescale(st, blk_max(s), c, rescale_raw);
    bf16x8 pf[2];
    exp_blk(st, s, c, neg_mc, pf);
    const lds_u8* vr[4];
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) vr[bd] = vread0[bd] + stg * kTileBytes;
    pv_blk(st, vr, 0, pf);
    // tile j+1 must have landed; with three stages tile j+2's four copies
    // may still fly
    if (NS > 2 && issue) sync_tiles<4>();
    else sync_tiles<0>();
    stg = stg == NS - 1 ? 0 : stg + 1;
  };

  // Start-up.  With the rotation in registers (RH >= 0) the first two K'/V
  // tiles, and on a gated windowed layer the gate rows, are requested before
  // the query rows so their latencies overlap; the generic rotation needs LDS
  // first.
  // Global layers: pair j holds tiles t_hi - 2j and t_hi - 2j - 1 in tile
  // stages 2 (j % 4) and 2 (j % 4) + 1.  An odd tile count ends with tile
  // -1: it is loaded from tile 0 (finite values) and masked out entirely.
  const int np = (nt + 1) / 2;
  auto gload_pair = [&](int j) {
    const int ps = j & 3;
    gload(t_hi - 2 * j, 2 * ps);
    gload(max(t_hi - 2 * j - 1, 0), 2 * ps + 1);
  };
  auto first_loads = [&] {
    if (BANDED) {
      gload(t_hi, 0);
      if (nt > 1) gload(t_hi - 1, 1);
    } else {
      gload_pair(0);
      if (np > 1) gload_pair(1);
    }
  };
  // Windowed layers move their query, gate and output rows in whole 256-byte
  // rows (16 lanes per row): each wave's 32 query rows go straight to LDS,
  // and lane L prefetches 8 gate values of row 4k + L/16 (k = 0..7) in the
  // layout of the coalesced output stores.
  const int wrow0 = i0w + (wv / geo.heads_per_wg) * 32;  // this wave's first query row
  const bool gate_pre = BANDED && p.gate != nullptr;
  u32x4 gco[8];
  if (BANDED) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int row = 4 * n + (lane >> 4);
      const long long qr = (tok0 + min(wrow0 + row, S - 1)) * p.Hq + head;
      dma16(p.q + qr * kD + 8 * ((lane & 15) ^ (row & 15)),
            lds_addr(smem + kQRegion + wvu * 32 * kRowBytes + n * 1024));
    }
  }
  if (BANDED || RH >= 0) first_loads();
  if (gate_pre) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const long long gr = (tok0 + min(wrow0 + 4 * k + (lane >> 4), S - 1)) * p.Hq + head;
      gco[k] = ld16(p.gate + gr * kD + 8 * (lane & 15));
    }
  }
  // ---- fused query prologue: RMSNorm (+ weight), partial RoPE, -> bf16 B operand
  {
    float x[64];
    if (BANDED) {
      // this wave's 32 query rows arrived in LDS (row q%32, chunks swizzled
      // by row); wait for them: the loads issued after them (4 per tile, 8
      // of gate) may still fly
      if (nt > 1) {
        if (gate_pre) wait_vm<16>();
        else wait_vm<8>();
      } else {
        if (gate_pre) wait_vm<12>();
        else wait_vm<4>();
      }
      const lds_u8* qr = smem + kQRegion + wv * 32 * kRowBytes + qcol * kRowBytes;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 v = lds_read_b128(qr + (((8 * half + j) ^ (qcol & 15)) << 4));
        unpack_bf16x8(__builtin_bit_cast(u32x4, v), x + 8 * j);
      }
    } else {
      const uint16_t* src = p.q + qrow * kD + 64 * half;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 u = qok ? ld16(src + 8 * j) : u32x4{0, 0, 0, 0};
        unpack_bf16x8(u, x + 8 * j);
      }
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
    if (RH > 0 && half == 0) {
      // rotary pairs (t, t + RH), all in this lane's registers
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
    } else if (RH < 0 && p.rope_half > 0 && half == 0) {
      // any rope_dim <= 64: the rotary dims live in the lane-half-0 registers;
      // go through a private LDS row so the partner dim is addressable
      // (windowed layers: behind the tiles in flight, in the wave's own query rows' region,
      // which it has already read)
      float* qs = reinterpret_cast<float*>(smem_raw + (BANDED ? kQRegion + wv * 32 * kRowBytes : 0)) +
                  (BANDED ? qcol * 64 : (wv * 32 + qcol) * 65);
#pragma unroll
      for (int d = 0; d < 64; ++d) qs[d] = x[d];
      const long long pos = p.pos_offset + qi;
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
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = pack_bf16x8(x + 8 * kk);
  }
  if (!BANDED && RH < 0) {
    __syncthreads();  // the prologue's LDS rows are reused by the KV tiles
    first_loads();
  }
  // tile 0 must have landed (loads issued after it: tile 1's copies, and on
  // gated windowed layers the eight gate rows)
  constexpr int kCopies = Cfg<BANDED>::kCopies;
  if (BANDED && gate_pre) {
    if (nt > 1) sync_tiles<kCopies + 8>();
    else sync_tiles<8>();
  } else if (BANDED) {
    if (nt > 1) sync_tiles<kCopies>();
    else sync_tiles<0>();
  } else {
    // pair 0 (pair 1's copies may fly)
    if (np > 1) sync_tiles<2 * kCopies>();
    else sync_tiles<0>();
  }
  if constexpr (BANDED) {
    for (int j = 0; j < nt; ++j) step(j, std::true_type{});
  } else {
    // Global layers: the two waves on each SIMD (w and w + 4) take turns,
    // on pairs of 32-key tiles.  Every wave runs the same sequence of phases
    // separated by barriers: softmax phase j (scores of pair j -> P) and
    // MFMA phase j (PV of pair j and QK' of pair j + 1, interleaved so that
    // each group of LDS operand reads flies under the previous eight
    // MFMAs).  Wave w + 4 passes one extra barrier first and wave w one
    // extra at the end, so that one runs its MFMA phase while the other runs
    // its softmax phase.
    //
    // Pair j + 2 is copied into the stage of pair j - 2 at the top of softmax
    // phase j: the other wave of the SIMD is then in MFMA phase j - 1, which
    // reads pairs j - 1 and j only.  Barriers after an MFMA phase wait for
    // every copy in flight (pair j + 2), those after a softmax phase for all
    // but the copies just issued, so pair j + 1 has landed for every wave
    // before the barrier that opens either wave's MFMA phase j.
    const bool second = wvu >= 4;
    bf16x8 ka[8], va[8], pf[4];
    f32x16 sa, sb;
    auto kstage = [&](int j, int u) { return smem + (2 * (j & 3) + u) * kTileBytes; };
    auto vops = [&](int j, int u) {
      const lds_u8* vr[4];
#pragma unroll
      for (int bd = 0; bd < 4; ++bd) vr[bd] = vread0[bd] + (2 * (j & 3) + u) * kTileBytes;
      load_vops(va, vr);
    };
    auto pv2 = [&](int t) {  // PV of one tile of the pair: P in pf[2t], pf[2t+1]
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int bd = 0; bd < 4; ++bd)
          st.acc[bd] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[4 * kt + bd], pf[2 * t + kt], st.acc[bd], 0, 0, 0);
      }
    };
    auto s_phase = [&](int j) {
      const int ta = t_hi - 2 * j, tb = ta - 1;
      if (ta * kBN + kBN - 1 > wrow0) mask_blk(sa, ta * kBN, qm, lim, half);
      if (tb < 0 || tb * kBN + kBN - 1 > wrow0) mask_blk(sb, tb * kBN, qm, lim, half);
      const float neg_mc = softmax_rescale(st, fmaxf(blk_max(sa), blk_max(sb)), c, rescale_raw);
      bf16x8 p2[2];
      exp_blk(st, sa, c, neg_mc, p2);
      pf[0] = p2[0];
      pf[1] = p2[1];
      exp_blk(st, sb, c, neg_mc, p2);
      pf[2] = p2[0];
      pf[3] = p2[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) pin(pf[i]);
      pin(st.l_run);
    };
    if (second) phase_barrier();
    // QK' of pair 0 and the V operands of its first tile
    load_kops(ka, kstage(0, 0), kread_off);
    qk_mfma(sa, ka, qf);
    __builtin_amdgcn_sched_barrier(0);
    load_kops(ka, kstage(0, 1), kread_off);
    qk_mfma(sb, ka, qf);
    vops(0, 0);
    phase_sync<0, false>();
    for (int j = 0; j < np; ++j) {
      if (j + 2 < np) gload_pair(j + 2);
      s_phase(j);
      if (j + 2 < np) phase_sync<2 * kCopies, true>();
      else phase_sync<0, true>();
      if (j + 1 < np) {
        load_kops(ka, kstage(j + 1, 0), kread_off);
        pv2(0);
        __builtin_amdgcn_sched_barrier(0);
        vops(j, 1);
        qk_mfma(sa, ka, qf);
        __builtin_amdgcn_sched_barrier(0);
        load_kops(ka, kstage(j + 1, 1), kread_off);
        pv2(1);
        __builtin_amdgcn_sched_barrier(0);
        vops(j + 1, 0);
        qk_mfma(sb, ka, qf);
        phase_sync<0, false>();
      }
    }
    pv2(0);
    __builtin_amdgcn_sched_barrier(0);
    vops(np - 1, 1);
    pv2(1);
    if (!second) phase_barrier();
  }

  // ---- epilogue: normalise, gate, store (register r of block bd, lane half
  // h -> dim 32 bd + 8 (r/4) + 4 h + r%4: four runs of 4 dims per block)
  const float l_tot = pair_sum32(st.l_run);
  const float inv = 1.0f / l_tot;
  if (p.lse && qok && half == 0)
    p.lse[lse0 + head * lse_hs + qi] = (st.m_run * c + __log2f(l_tot)) * kLn2;
  if (BANDED) {
    // fp32 rows to LDS (the tiles are dead: every wave passed the last
    // barrier), 16-byte chunk c of row q at chunk c ^ q; then row-coalesced
    // gate and store, lane L handling dims 8(L%16).. of row 4k + L/16.
    lds_u8* orow = smem + wv * 32 * 512;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st.acc[bd][4 * q4 + e] * inv;
        const int ch = 8 * bd + 2 * q4 + half;
        *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
            orow + qcol * 512 + ((ch ^ qcol) << 4)) = o;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 4 * k + (lane >> 4);
      const int ch0 = 2 * (lane & 15);
      const f32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          orow + row * 512 + ((ch0 ^ row) << 4));
      const f32x4 a2 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          orow + row * 512 + (((ch0 + 1) ^ row) << 4));
      float o[8] = {a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      if (gate_pre) {
        float gv[8];
        unpack_bf16x8(gco[k], gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= sigmoidf_(gv[e]);
      }
      if (wrow0 + row < S) {
        const long long orw = (tok0 + wrow0 + row) * p.Hq + head;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
        st16(p.out + orw * kD + 8 * (lane & 15), w);
      }
    }
  } else if (qok) {
    uint16_t* dst = p.out + qrow * kD + 4 * half;
    const uint16_t* gsrc = p.gate ? p.gate + qrow * kD + 4 * half : nullptr;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st.acc[bd][4 * q4 + e] * inv;
        const int off = 32 * bd + 8 * q4;
        if (gsrc) {
          const uint2 gg = *reinterpret_cast<const uint2*>(gsrc + off);
          o[0] *= sigmoidf_(bf_lo(gg.x));
          o[1] *= sigmoidf_(bf_hi(gg.x));
          o[2] *= sigmoidf_(bf_lo(gg.y));
          o[3] *= sigmoidf_(bf_hi(gg.y));
        }
        uint2 w;
        w.x = pack_bf16x2(o[0], o[1]);
        w.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(dst + off) = w;
      }
    }
  }
}

template <int RH, bool PACKED>
void launch_variant(bool banded, dim3 grid, dim3 block, hipStream_t stream, const FlashParams& p,
                    const Geo& geo) {
  if (banded)
    hipLaunchKernelGGL((flash_fwd_kernel<true, RH, PACKED>), grid, block, 0, stream, p, geo);
  else
    hipLaunchKernelGGL((flash_fwd_kernel<false, RH, PACKED>), grid, block, 0, stream, p, geo);
}

}  // namespace

hipError_t launch_flash_fwd(const FlashParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const int grp = p.Hq / p.Hkv;
  const bool banded = p.window > 0;
  const int waves = banded ? Cfg<true>::kWaves : Cfg<false>::kWaves;
  Geo geo;
  geo.heads_per_wg = grp < waves ? grp : waves;
  geo.hgroups = grp / geo.heads_per_wg;
  geo.pos_per_wg = 32 * waves / geo.heads_per_wg;
  geo.n_pos_blocks = (p.S + geo.pos_per_wg - 1) / geo.pos_per_wg;
  geo.n_bhg = p.B * p.Hkv * geo.hgroups;
  const long long blocks = (long long)geo.n_pos_blocks * geo.n_bhg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * waves);
  if (p.cu_seqlens) {
    if (p.rope_half == 21) launch_variant<21, true>(banded, grid, block, stream, p, geo);
    else if (p.rope_half == 0) launch_variant<0, true>(banded, grid, block, stream, p, geo);
    else launch_variant<-1, true>(banded, grid, block, stream, p, geo);
  } else {
    if (p.rope_half == 21) launch_variant<21, false>(banded, grid, block, stream, p, geo);
    else if (p.rope_half == 0) launch_variant<0, false>(banded, grid, block, stream, p, geo);
    else launch_variant<-1, false>(banded, grid, block, stream, p, geo);
  }
  return hipGetLastError();
}

}  // namespace zg
