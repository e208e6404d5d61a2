// Banded (sliding-window) flash attention, forward.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: a sliding-window layer
// lets each token attend only to its 128 neighbouring tokens.  Section
// 核心方法: GQA, 32 query heads share 8 KV heads.  Page "7B 打 235B？…全开源
// 配方" (shibing624.github.io), section 🏗️ 架构: the local attention output
// is multiplied by a sigmoid gate.  (The global layers run in
// flash_causal.hip.)
//
// A workgroup of four waves serves one KV head g and 32 query positions;
// each wave is one query head of g's group (GQA packing: every K'/V tile in
// LDS feeds all four waves).  Lane l owns query row l%32 and the half l/32
// of everything else, so the online softmax needs one cross-half exchange
// per tile and no other cross-lane traffic.
//
//   S^T = K' Q'^T  (v_mfma_f32_32x32x16_bf16, A = K' tile rows from LDS,
//                   B = the wave's normalised + rotated Q' in registers)
//   O^T += V^T P^T (A = V^T read from the row-major V tile with the gfx950
//                   transposing LDS load ds_read_b64_tr_b16, B = P in registers)
//
// K' and V tiles go from global memory straight into LDS (global_load_lds,
// no register staging) through a ring of three tile stages, row-major with
// 256-byte rows whose 16-byte chunks are XOR-swizzled by row: chunk ^ (row &
// 15) for K', chunk ^ ((row & 3) << 2) for V.  With the 64-bank LDS every
// MFMA operand read is then free of bank conflicts, and each read address is
// a per-lane base plus an immediate.
//
// Only KV tiles that intersect the band of the workgroup's queries are
// visited: ceil((32 + W - 1) / 32) + 1 tiles at most for a window W.  The
// query prologue (RMSNorm + partial RoPE, and the softmax scale times
// log2(e), so that scores come out in exp2 units) is fused into the Q load;
// the sigmoid gate is fused into the epilogue.  Softmax runs in fp32 with
// p = exp2(s - m) and lazy rescaling of the accumulator (only when the
// running max grows by more than 2^8).

#include <type_traits>

#include "zg_common.h"
#include "zg_launch.h"
#include "zg_lds.h"
#include "zg_flash_tile.h"

namespace zg {

namespace {

using namespace flash;

// Four waves per workgroup (the four query heads of a KV group at 32
// positions); each wave copies 2 KB of every K'/V tile.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlocksPerWave = 2;  // 1 KB blocks of each tile a wave copies
constexpr int kCopies = 4;         // its K' + V copies per tile
// LDS ring per K' and V, K' stages first, then the V stages: three tile
// stages, copies fly two tiles ahead; 48 KB in all, so that three
// workgroups fit a CU.  Before the loop the query rows (8 KB per wave) are
// staged in the stages tiles 1 and 2 will use: waves 0, 1 in K' stages 1, 2,
// waves 2, 3 in V stages 1, 2.  After the loop the fp32 output rows are
// staged in two halves of 64 dims (8 KB per wave per half) for coalesced
// stores.
constexpr int NS = 3;
constexpr int kVOff = NS * kTileBytes;
constexpr int kSmemBanded = 2 * NS * kTileBytes;  // 49152
constexpr int kOutHalfBytes = 32 * 64 * 4;        // a wave's 32 rows x 64 fp32
static_assert(kWaves * kOutHalfBytes <= kSmemBanded, "output staging must fit");
// this wave's query-row staging area (8 KB)
__device__ __forceinline__ int q_stage_off(int w) {
  return w < 2 ? (1 + w) * kTileBytes : kVOff + (w - 1) * kTileBytes;
}

// The query, gate and output rows are touched once, so they move with the
// non-temporal hint and leave L2 to the K'/V tiles that the neighbouring
// query blocks share (B4 S4096 with cold caches: 0.155-0.159 -> 0.137-0.140
// ms; 256K layer -2%).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
// dma16 with the non-temporal hint
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds)
               : "memory");
}

// RH: rope_dim / 2 when known at compile time (0 or 21: the rotation runs in
// registers), -1 for any other rope_dim (rotation through LDS).
template <int RH, bool PACKED>
__global__ __launch_bounds__(kThreads, 3) void flash_fwd_kernel(FlashParams p, Geo geo) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmemBanded];
  lds_u8* smem = (lds_u8*)smem_raw;  // generic -> LDS address space

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int qcol = lane & 31;
  const int half = lane >> 5;
  const int grp = p.Hq / p.Hkv;

  // ---- workgroup -> (position block, batch, kv head, head group)
  const int bid = blockIdx.x;
  const int bhg = bid % geo.n_bhg;
  const int pb = bid / geo.n_bhg;
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
  // wave-wide lazy-rescale vote is that of a real row.
  const int qm = min(qi, S - 1);
  const int lim = min(p.window, qm + 1);
  const int hi = min(S, i0w + geo.pos_per_wg);  // keys < hi
  const int lo = max(0, i0w - p.window + 1);    // keys >= lo

  bf16x8 qf[8];  // this wave's Q' rows: the B operand of every S MFMA

  // ---- KV tile staging: global -> LDS directly (global_load_lds_dwordx4)
  // into a ring of NS stages, so that a tile's loads have NS - 1 tiles of
  // compute to arrive.  Wave wv fills the BPW 1 KB blocks BPW wv + j (rows
  // 4n..4n+3) of each 8 KB tile: lane L writes physical chunk L%16 of row
  // 4n + L/16 and so fetches the logical chunk that the row's swizzle places
  // there.
  constexpr int BPW = kBlocksPerWave;
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
  // Q' carries the softmax scale times log2(e): scores are in exp2 units
  const float c = 1.0f;
  const float rescale_raw = kRescaleThreshold;
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
  // t = t_hi - j holds keys [32t, 32t + 32); every tile is masked.
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

  // Start-up: the query rows and the first K'/V tile are requested together,
  // so their latencies overlap; tile 1 follows once every wave has read its
  // query rows out of tile 1's stage.  The query, gate and output rows move
  // in whole rows: each wave's 32 query rows go straight to LDS (16 lanes per
  // 256-byte row); after the loop lane L loads 8 gate values of row
  // 8k + L/8 (k = 0..3), dims 64 r + 8 (L%8) (r = 0, 1), the layout of the
  // coalesced output stores (held from the start they would cost 32
  // registers, which three workgroups per CU do not leave).
  const int wrow0 = i0w + (wv / geo.heads_per_wg) * 32;  // this wave's first query row
  const bool gate_pre = p.gate != nullptr;
  const int qoff = q_stage_off(wvu);
  u32x4 gco[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int row = 4 * n + (lane >> 4);
    const long long qr = (tok0 + min(wrow0 + row, S - 1)) * p.Hq + head;
    dma16_nt(p.q + qr * kD + 8 * ((lane & 15) ^ (row & 15)), lds_addr(smem + qoff + n * 1024));
  }
  gload(t_hi, 0);
  // ---- fused query prologue: RMSNorm (+ weight), partial RoPE, -> bf16 B operand
  {
    float x[64];
    // this wave's 32 query rows arrived in LDS (row q%32, chunks swizzled by
    // row); wait for them: the loads issued after them (tile 0's 4, 8 of
    // gate) may still fly
    wait_vm<4>();
    const lds_u8* qr = smem + qoff + qcol * kRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 v = lds_read_b128(qr + (((8 * half + j) ^ (qcol & 15)) << 4));
      unpack_bf16x8(__builtin_bit_cast(u32x4, v), x + 8 * j);
    }
    // (the generic rotation goes through a private LDS row per lane, in the
    // wave's own query rows' region, which it has already read, behind the
    // tiles in flight)
    float* qs = reinterpret_cast<float*>(smem_raw + qoff) + qcol * 64;
    q_prologue<RH>(x, half, p, p.pos_offset + qi, qs, qf, p.q_norm_w);
  }
  // every wave has read its query rows: tile 1 may take its stage
  lds_barrier();
  if (nt > 1) gload(t_hi - 1, 1);
  // tile 0 must have landed (tile 1's copies may fly)
  if (nt > 1) sync_tiles<kCopies>();
  else sync_tiles<0>();
  for (int j = 0; j < nt; ++j) step(j, std::true_type{});
  // the gate rows, in the layout of the coalesced output stores
  if (gate_pre) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const long long gr = (tok0 + min(wrow0 + 8 * k + (lane >> 3), S - 1)) * p.Hq + head;
        gco[4 * r + k] = ld16_nt(p.gate + gr * kD + 64 * r + 8 * (lane & 7));
      }
    }
  }

  // ---- epilogue: normalise, gate, store (register r of block bd, lane half
  // h -> dim 32 bd + 8 (r/4) + 4 h + r%4: four runs of 4 dims per block)
  const float l_tot = pair_sum32(st.l_run);
  const float inv = 1.0f / l_tot;
  if (p.lse && qok && half == 0)
    p.lse[lse0 + head * lse_hs + qi] = (st.m_run * c + __log2f(l_tot)) * kLn2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    // dims 64 r .. 64 r + 63 of the fp32 rows to LDS (the tiles are dead:
    // every wave passed the last barrier; each wave uses its own 8 KB, in
    // program order, so no barrier is needed between the halves): 16-byte
    // chunk c of row q at chunk c ^ (q % 16); then row-coalesced gate and
    // store, lane L handling dims 64 r + 8 (L%8).. of row 8k + L/8.
    lds_u8* orow = smem + wv * kOutHalfBytes;
#pragma unroll
    for (int bh = 0; bh < 2; ++bh) {
      const int bd = 2 * r + bh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st.acc[bd][4 * q4 + e] * inv;
        const int ch = 8 * bh + 2 * q4 + half;
        *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
            orow + qcol * 256 + ((ch ^ (qcol & 15)) << 4)) = o;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = 8 * k + (lane >> 3);
      const int ch0 = 2 * (lane & 7);
      const f32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          orow + row * 256 + ((ch0 ^ (row & 15)) << 4));
      const f32x4 a2 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          orow + row * 256 + (((ch0 + 1) ^ (row & 15)) << 4));
      float o[8] = {a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      if (gate_pre) {
        float gv[8];
        unpack_bf16x8(gco[4 * r + k], gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= sigmoidf_(gv[e]);
      }
      if (wrow0 + row < S) {
        const long long orw = (tok0 + wrow0 + row) * p.Hq + head;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
        st16_nt(p.out + orw * kD + 64 * r + 8 * (lane & 7), w);
      }
    }
  }
}

template <int RH, bool PACKED>
void launch_variant(dim3 grid, hipStream_t stream, const FlashParams& p, const Geo& geo) {
  hipLaunchKernelGGL((flash_fwd_kernel<RH, PACKED>), grid, dim3(kThreads), 0, stream, p, geo);
}

}  // namespace

hipError_t launch_flash_fwd(const FlashParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  if (p.window <= 0) return launch_flash_causal(p, stream);
  const int grp = p.Hq / p.Hkv;
  Geo geo;
  geo.heads_per_wg = grp < kWaves ? grp : kWaves;
  geo.hgroups = grp / geo.heads_per_wg;
  geo.pos_per_wg = 32 * kWaves / geo.heads_per_wg;
  geo.n_pos_blocks = (p.S + geo.pos_per_wg - 1) / geo.pos_per_wg;
  geo.n_bhg = p.B * p.Hkv * geo.hgroups;
  const long long blocks = (long long)geo.n_pos_blocks * geo.n_bhg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (p.cu_seqlens) {
    if (p.rope_half == 21) launch_variant<21, true>(grid, stream, p, geo);
    else if (p.rope_half == 0) launch_variant<0, true>(grid, stream, p, geo);
    else launch_variant<-1, true>(grid, stream, p, geo);
  } else {
    if (p.rope_half == 21) launch_variant<21, false>(grid, stream, p, geo);
    else if (p.rope_half == 0) launch_variant<0, false>(grid, stream, p, geo);
    else launch_variant<-1, false>(grid, stream, p, geo);
  }
  return hipGetLastError();
}

}  // namespace zg
