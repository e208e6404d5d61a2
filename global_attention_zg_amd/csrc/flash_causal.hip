// Global (full causal) flash attention, forward.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: the global layers
// attend over the whole causal prefix; section 核心方法: GQA, 32 query heads
// share 8 KV heads.  Section 技术新颖性: the quadratic cost of these layers is
// what the hybrid's advantage at long context comes from, so this kernel is
// where a long prefill spends its time.
//
// One wave per SIMD.  A workgroup of four waves serves one KV head g and 64
// query positions: wave w is query head w of g's group at all 64 positions
// (GQA packing: each K'/V tile copied into LDS feeds the four heads).  A wave
// holds its 64 query rows as two halves of 32 rows, each with its own
// accumulator (128 fp32 per lane in all), so that every K' and V operand it
// reads from LDS feeds two MFMAs.
//
// Per 32-key tile the wave runs four slots; the MFMAs of each slot do not
// depend on the VALU work placed beside them, so the matrix cores and the
// vector ALUs of the SIMD work side by side:
//   A: S0 = K'(j+1) Q0'^T           beside  softmax of half 1 on tile j -> P1
//   B: O1 += V(j)^T P1^T             beside  softmax of half 0 on tile j+1 -> P0
//   C: S1 = K'(j+1) Q1'^T           beside  the V(j+1) operand reads
//   D: O0 += V(j+1)^T P0^T           beside  the K'(j+2) operand reads
// No running max: each row's softmax offset is a bound on its scores taken
// from the QK-RMSNorm (see the prologue), so P = exp2(s - U) needs neither a
// max nor a rescale; a workgroup whose rows could underflow under that bound
// first takes the exact row maxima in a scores-only pass.
//
// K'/V tiles go global -> LDS directly (global_load_lds_dwordx4) through a
// ring of NS tile stages with the banded kernel's swizzled 256-byte rows;
// copies fly NS - 2 tiles ahead, and one barrier per tile both publishes the
// tile two ahead and frees the stage of the tile just read.  Tiles are
// visited from the diagonal down.
//
// The grid is persistent: one workgroup per CU takes jobs (query blocks,
// longest causal rows first) from per-XCD work queues (zg_queue.h) until all
// are empty, so that XCDs running at different speeds finish together.
//
// The E4M3 variant (page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型",
// section 前置知识 › FP8 混合精度训练与 TWEO: forward matrix multiplies in
// E4M3 with power-of-two scaling) runs S = K' Q'^T on the FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, two per 32-key block and 32 query rows):
// K' arrives as E4M3 codes of K' * k_scale (128-byte LDS rows), each query
// row is quantized with its own power-of-two scale in the prologue, and the
// softmax multiplies the code products by c / (query scale * k_scale) in the
// same FMA that subtracts the row's offset.  P V stays in bf16.

#include <algorithm>
#include <type_traits>

#include "zg_common.h"
#include "zg_fp8.h"
#include "zg_launch.h"
#include "zg_lds.h"
#include "zg_flash_tile.h"
#include "zg_queue.h"

namespace zg {

namespace {

using namespace flash;

constexpr int kCWaves = 4;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kCRows = 64;       // query rows per wave (two halves of 32)

// Causal mask of one 32-key block for this lane's row: register r holds key
// kblk + 4 h + 8 (r/4) + r%4, visible iff key <= qm, i.e. iff the immediate
// 8 (r/4) + r%4 is at most thr = qm - kblk - 4 h.
__device__ __forceinline__ void mask_causal(f32x16& s, int thr) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) > thr ? -INFINITY : s[r];
}

// S^T = K' Q'^T + seed for one 32-key block: Q' carries the softmax scale
// times log2(e) and the accumulator starts from minus the row's softmax
// offset, so the result is the exp2 argument of P itself.
__device__ __forceinline__ void qk_seeded(f32x16& s, const bf16x8 (&ka)[8], const bf16x8 (&qf)[8],
                                          const f32x16& seed) {
  s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], seed, 0, 0, 0);
#pragma unroll
  for (int kk = 1; kk < 8; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s, 0, 0, 0);
}

// A word of P: two elements exp2(a0), exp2(a1) packed to bf16 (a word of
// the PV B operand), and their sum, from the rounded values the MFMA
// multiplies, added to the row sum.
__device__ __forceinline__ uint32_t p_word(float a0, float a1, float& l_run) {
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  const uint32_t u = pack_bf16x2(fast_exp2(a0), fast_exp2(a1));
  l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u), one2, l_run, false);
  return u;
}

// O^T += V^T P^T (the operand layout of load_vops and P) with the accumulator held
// in AGPRs by the asm constraint, so that the register allocator never moves
// it; the score MFMAs then write their results to VGPRs, where the softmax
// reads them.  Back-to-back accumulation into the same registers needs no
// wait states; a VALU read of the accumulator does (acc_settle).
__device__ __forceinline__ void pv_agpr(f32x16 (&acc)[4], const bf16x8 (&va)[8],
                                        const bf16x8 (&pf)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[bd]) : "v"(va[4 * t + bd]), "v"(pf[t]));
  }
}

// The i-th MFMA (k-step i/4, dim block i%4) of pv_agpr.
__device__ __forceinline__ void pv_agpr_one(f32x16 (&acc)[4], const bf16x8 (&va)[8],
                                            const bf16x8 (&pf)[2], int i) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[i % 4]) : "v"(va[i]), "v"(pf[i / 4]));
}

// Wait states between the last accumulation and a VALU read of the
// accumulator (more than the 18 an MFMA of 16 passes needs).
__device__ __forceinline__ void acc_settle(f32x16 (&acc)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
}

// S^T = K' Q'^T of one 32-key block on the FP8 matrix cores: operand m holds
// dims 64 h + 32 m .. + 31 (h = lane / 32) as E4M3 codes, the same dims for
// the key row (A) and the query row (B), so the products pair up whatever
// order the unit sums them in.  The block scales are 1: the result is the sum
// of the code products.
__device__ __forceinline__ void qk_fp8(f32x16& s, const i32x8 (&ka)[2], const i32x8 (&qf)[2]) {
  s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[0], qf[0], f32x16{}, 0, 0, 0, 127, 0, 127);
  s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[1], qf[1], s, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join_i32x8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// RH: rope_dim / 2 when fixed at compile time (21 or 0), else -1.
// NS: K'/V tile stages in LDS.  FP8: the E4M3 variant.  ILV: the V operand
// reads are interleaved with the second half's score MFMAs, in groups of
// ILV MFMAs and 2 * ILV reads (0: not interleaved).  Interleaving is 2-4%
// faster up to 64K keys and 3% at 256K since the grid is persistent; groups
// of two are 0.5-0.8% faster again at 256K (0.3% slower at 64K); the E4M3
// variant keeps the plain schedule above 64K keys, where both run alike.
template <int RH, bool PACKED, int NS, bool FP8, int ILV>
__global__ __launch_bounds__(kCThreads, 1) void flash_causal_kernel(FlashParams p, Geo geo) {
  constexpr int kKRow = FP8 ? kD : kRowBytes;  // bytes per K' row in LDS
  constexpr int kKTile = kBN * kKRow;
  constexpr int kSmem = NS * (kKTile + kTileBytes);
  constexpr int kVOff = NS * kKTile;
  // a wave's global -> LDS copies per tile: 2 KB of V and 2 KB (bf16) or
  // 1 KB (E4M3) of K'
  constexpr int kCopies = FP8 ? 3 : 4;
  constexpr int kKOps = FP8 ? 2 : 8;  // score-product operands per 32 rows
  constexpr int kQkMfma = kKOps;      // score MFMAs per 32 rows and 32 keys
  using QOp = typename std::conditional<FP8, i32x8, bf16x8>::type;
  static_assert(kCWaves * 32 * 65 * 4 <= kSmem, "query RoPE rows must fit");
  static_assert(NS >= 3, "copies fly NS - 2 tiles ahead");
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmem];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int qcol = lane & 31;
  const int half = lane >> 5;
  const int grp = p.Hq / p.Hkv;

  __shared__ int job_s[2];  // the next job, one slot per parity of the job loop
  __shared__ __attribute__((aligned(16))) float qw_s[kD];  // query-norm weights
  if (tid < kD / 4) st16(qw_s + 4 * tid, ld16(p.q_norm_w + 4 * tid));  // (published by the job loop's barrier)
  // max |w_k| over the 128 key-norm weights (two per lane, then the wave)
  float wk = fmaxf(fabsf(p.k_norm_w[2 * lane]), fabsf(p.k_norm_w[2 * lane + 1]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wk = fmaxf(wk, __shfl_xor(wk, o));
  const int own = blockIdx.x % geo.nq;  // this workgroup's own queue
  bool own_done = false;

  // One job: query block pb of (batch, kv head, head group) bhg, numbered
  // longest causal rows first.  Wave 0 claims the workgroup's next job into
  // `next`: the ticket is taken once the job's tiles are done and read after
  // the epilogue, so that the claim's latency hides under it, and the
  // workgroups that finish first take the longest jobs left.
  auto run_job = [&](const int bid, int& next) __attribute__((always_inline)) {
  // ---- job -> (position block, batch, kv head, head group)
  const int bhg = bid % geo.n_bhg;
  const int pb = geo.n_pos_blocks - 1 - bid / geo.n_bhg;  // longest causal rows first
  const int hg = bhg % geo.hgroups;
  const int bgi = bhg / geo.hgroups;
  const int g = bgi % p.Hkv;
  const int b = bgi / p.Hkv;
  const int head = g * grp + hg * geo.heads_per_wg + (wv % geo.heads_per_wg);
  const int i0w = pb * geo.pos_per_wg;
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
    if (i0w >= S) {  // whole workgroup: past the end of a short sequence
      if (wv == 0)
        next = next_job(p.queue, own, geo.nq, geo.n_jobs, own_done,
                        __builtin_amdgcn_readfirstlane(claim_own(p.queue, own, own_done)));
      return;
    }
  }
  // This wave's rows: half h is rows wrow0 + 32 h + (lane % 32).  Rows past
  // the end are padding with row S-1's visibility.
  const int wrow0 = i0w + (wv / geo.heads_per_wg) * kCRows;
  int qi[2], qm[2];
  bool qok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    qi[h] = wrow0 + 32 * h + qcol;
    qok[h] = qi[h] < S;
    qm[h] = min(qi[h], S - 1);
  }
  const int hi = min(S, i0w + geo.pos_per_wg);  // keys < hi
  const int t_hi = (hi - 1) / kBN;
  const int nt = t_hi + 1;

  // ---- K'/V staging: wave w fills the 1 KB blocks 2w, 2w + 1 (rows 4n ..
  // 4n + 3) of each 8 KB tile; lane L writes physical chunk L % 16 of row
  // 4n + L / 16 and so fetches the logical chunk the row's swizzle puts there.
  // E4M3 K' (4 KB tiles of 128-byte rows; chunk c of row r at physical chunk
  // c ^ ((r / 2) % 8), so that the 16 rows one 16-lane read group touches
  // cover all 64 banks): wave w fills rows 8w .. 8w + 7, lane L physical
  // chunk L % 8 of row 8w + L / 8.
  const long long kvstride = (long long)p.Hkv * kD;  // elements per token
  constexpr int kKEB = FP8 ? 1 : 2;                  // bytes per K' element
  const unsigned char* kbase =
      FP8 ? p.kp8 + tok0 * kvstride + g * kD
          : reinterpret_cast<const unsigned char*>(p.kp + tok0 * kvstride + g * kD);
  const uint16_t* vbase = p.v + tok0 * kvstride + g * kD;
  const int krow8 = 8 * wv + (lane >> 3);
  const uint32_t krow8_off = (uint32_t)(krow8 * kvstride);
  const uint32_t kchunk8 = 16u * ((lane & 7) ^ ((krow8 >> 1) & 7));
  uint32_t row_off[2], kchunk[2];
  int lrow[2];
  const uint32_t vchunk = 16u * ((lane & 15) ^ (((lane >> 4) & 3) << 2));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lrow[j] = 4 * (2 * wv + j) + (lane >> 4);
    row_off[j] = (uint32_t)(lrow[j] * kvstride * 2);
    kchunk[j] = 16u * ((lane & 15) ^ (lrow[j] & 15));
  }
  // tile t (0 <= t <= t_hi) -> stage stg; keys >= S (only in the top tile)
  // load key S-1 and are masked out
  auto gload = [&](int t, int stg) __attribute__((always_inline)) {
    const unsigned char* kb = kbase + (long long)t * kBN * kvstride * kKEB;
    const unsigned char* vb = (const unsigned char*)(vbase + (long long)t * kBN * kvstride);
    const uint32_t kl = lds_addr(smem + stg * kKTile + (FP8 ? 1 : 2) * wv * 1024);
    const uint32_t vl = lds_addr(smem + kVOff + stg * kTileBytes + 2 * wv * 1024);
    if (t * kBN + kBN <= S) {
      if constexpr (FP8) dma16_s(kb, krow8_off + kchunk8, kl);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (!FP8) dma16_s(kb, row_off[j] + kchunk[j], kl + j * 1024);
        dma16_s(vb, row_off[j] + vchunk, vl + j * 1024);
      }
    } else {
      if constexpr (FP8)
        dma16_s(kb, (uint32_t)((min(t * kBN + krow8, S - 1) - t * kBN) * kvstride) + kchunk8, kl);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t off = (uint32_t)((min(t * kBN + lrow[j], S - 1) - t * kBN) * kvstride * 2);
        if constexpr (!FP8) dma16_s(kb, off + kchunk[j], kl + j * 1024);
        dma16_s(vb, off + vchunk, vl + j * 1024);
      }
    }
  };
  // visit index j -> tile t_hi - j; indices past the last tile copy tile 0
  // (finite values, never used), which keeps the number of copies in flight
  // the same on every iteration
  auto gload_j = [&](int j, int stg) __attribute__((always_inline)) { gload(max(t_hi - j, 0), stg); };

  // per-lane LDS read offsets: K' row q%32 at logical chunk 8h (E4M3: 4h);
  // V rows 4h + i/4 at dims 32bd + 16 (group parity) + 4 (i%4) for the
  // transposing loads
  const uint32_t kread_off =
      FP8 ? qcol * kKRow + ((uint32_t)((4 * half) ^ ((qcol >> 1) & 7)) << 4)
          : qcol * kRowBytes + ((uint32_t)((8 * half) ^ (qcol & 15)) << 4);
  const int gi = lane & 15;
  const int vq = gi >> 2;
  const int vlow = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
  const lds_u8* vread0[4];  // stage 0; stage k adds k * kTileBytes
#pragma unroll
  for (int bd = 0; bd < 4; ++bd) {
    const int off = (4 * half + vq) * kRowBytes + (((bd ^ vq) << 2 | vlow) << 4) + 8 * (gi & 1);
    vread0[bd] = smem + kVOff + off;
  }

  TileState st[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) st[h].acc[bd] = f32x16{};
    st[h].l_run = 0.f;
  }

  // ---- start-up: the ring is filled with the first NS tiles while the
  // query rows are loaded and normalised + rotated (the generic rotation uses
  // LDS rows first and fills the ring afterwards)
  auto fill_ring = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < NS; ++jj) gload_j(jj, jj);
  };
  // Both halves' query rows are loaded first and the ring copies issued
  // after them, so that one round trip brings them all.
  u32x4 qraw[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const long long qrow = (tok0 + (qok[h] ? qi[h] : 0)) * p.Hq + head;
    const uint16_t* src = p.q + qrow * kD + 64 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j) qraw[h][j] = ld16(src + 8 * j);  // (rows past the end: row 0, zeroed below)
  }
  if (RH >= 0) fill_ring();
  QOp qf[2][kKOps];
  float fsc[2] = {1.f, 1.f};  // E4M3: exp2 units per unit of code product, per half
  bool fast_ok = true;
  // (the halves are fenced from each other so that the scheduler does not
  // overlap their work: the register peak of the prologue would otherwise
  // push the loop's operands out to scratch)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __builtin_amdgcn_sched_barrier(0);
    float x[64];
#pragma unroll
    for (int j = 0; j < 8; ++j) unpack_bf16x8(qok[h] ? qraw[h][j] : u32x4{0, 0, 0, 0}, x + 8 * j);
    float* qs = reinterpret_cast<float*>(smem_raw) + (wv * 32 + qcol) * 65;
    float qq = 0.f, u;
    if constexpr (FP8) {
      // E4M3 query row: q' with the power-of-two scale 2^(8-e) that puts its
      // amax = m 2^e (m in [0.5, 1), e clamped to >= -100) in [128, 256)
      q_norm_rope<RH>(x, half, p, p.pos_offset + qi[h], qs, qw_s);
      float am = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) am = fmaxf(am, fabsf(x[d]));
      am = pair_max32(am);
      int e;
      frexpf(am, &e);
      e = max(e, -100);
      uint2 c8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c8[j] = pack_e4m3x8(x + 8 * j, ldexpf(1.0f, 8 - e));
#pragma unroll
      for (int m = 0; m < 2; ++m)
        qf[h][m] = join_i32x8(u32x4{c8[4 * m].x, c8[4 * m].y, c8[4 * m + 1].x, c8[4 * m + 1].y},
                              u32x4{c8[4 * m + 2].x, c8[4 * m + 2].y, c8[4 * m + 3].x, c8[4 * m + 3].y});
      fsc[h] = p.scale_log2 * ldexpf(1.0f / p.k_scale, e - 8);
      // |codes| of the row and its product with the row's own key's codes
      const unsigned char* krow = p.kp8 + ((tok0 + qm[h]) * p.Hkv + g) * kD + 64 * half;
      float sii = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float qv[8], kv[8];
        unpack_bf16x8(widen_e4m3x8(c8[j]), qv);
        unpack_bf16x8(widen_e4m3x8(ld8(krow + 8 * j)), kv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          qq = __builtin_fmaf(qv[i], qv[i], qq);
          sii = __builtin_fmaf(qv[i], kv[i], sii);
        }
      }
      qq = pair_sum32(qq);
      sii = pair_sum32(sii) * fsc[h];
      // Softmax offset (exp2 units): every score is at most fsc |q codes|
      // |k codes| by Cauchy-Schwarz, and a key row's codes have norm at most
      // k_scale |k'| (1 + 2^-4) + 2^-10 sqrt(D) (relative rounding 2^-4 of
      // normal values, 2^-10 absolute below them; clamping only shrinks
      // them), with |k'| <= sqrt(D) max|w_k|; 2^-8 covers the fp32 sums.
      const float kc_norm = (p.k_scale * wk * 1.0625f + 0.0009765625f) * sqrtf((float)kD);
      u = fsc[h] * sqrtf(qq) * kc_norm * (1.0f + 0.00390625f);
      fast_ok = fast_ok && u - sii <= 100.0f;
    } else {
      q_prologue<RH>(x, half, p, p.pos_offset + qi[h], qs, qf[h], qw_s);
    // Softmax offset.  q' is held pre-scaled by c = scale log2(e), so the
    // scores come out in exp2 units.  Every score of this row is at most
    //   U = |c q'| sqrt(D) max|w_k|   (RoPE keeps norms; the key RMSNorm
    // bounds each normalised key by sqrt(D) before the weight), taken here
    // over the bf16 c q' the products use and widened by 2^-6 for the bf16
    // rounding of k' and the fp32 sums.  With P = exp2(s - U) every weight is
    // at most 1.  The row's own key is visible, so its largest weight is at
    // least exp2(s_ii - U); while that stays above 2^-100 the fixed offset
    // loses nothing to underflow and no running max is needed (s_ii is taken
    // below, once the ring holds the row's own key).
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float qv[8];
        unpack_bf16x8(__builtin_bit_cast(u32x4, qf[h][j]), qv);
#pragma unroll
        for (int e = 0; e < 8; ++e) qq = __builtin_fmaf(qv[e], qv[e], qq);
      }
      qq = pair_sum32(qq);
      u = sqrtf(qq) * sqrtf((float)kD) * wk * (1.0f + 0.015625f);
    }
    st[h].m_run = u;
    // the query operands stay in accumulation registers for the whole
    // kernel (the matrix cores read their A/B operands from either file),
    // which leaves the vector registers to the loop's working set
#pragma unroll
    for (int kk = 0; kk < kKOps; ++kk) asm volatile("; q' operand to AGPRs" : "=a"(qf[h][kk]) : "0"(qf[h][kk]));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (RH < 0) {
    lds_barrier();  // every wave is done with its rotation rows
    fill_ring();
  }
  sync_tiles<0>();
  if constexpr (!FP8) {
    // s_ii from the ring: the row's own key is in the tile of visit
    // t_hi - qm / 32, which sits in the stage of that number (< NS: a
    // workgroup covers at most 256 positions), row qm % 32, logical chunk c
    // at physical chunk c ^ (row % 16)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tk = qm[h] / kBN;
      const int r = qm[h] - tk * kBN;
      const lds_u8* kr = smem + (t_hi - tk) * kKTile + r * kRowBytes;
      float sii = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float qv[8], kv[8];
        unpack_bf16x8(__builtin_bit_cast(u32x4, qf[h][j]), qv);
        unpack_bf16x8(__builtin_bit_cast(u32x4, lds_read_b128(kr + ((uint32_t)((8 * half + j) ^ (r & 15)) << 4))), kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) sii = __builtin_fmaf(qv[e], kv[e], sii);
      }
      sii = pair_sum32(sii);
      fast_ok = fast_ok && st[h].m_run - sii <= 100.0f;
    }
  }
  // Workgroup-uniform: if any row's largest weight could underflow, every
  // wave first takes its rows' exact maxima (a pass of the score products
  // alone) and uses those as the offsets instead.
  const bool exact_max = __syncthreads_or(!fast_ok) != 0;

  // a tile needs masking for half h if it reaches past the half's first row
  auto masked = [&](int j, int h) __attribute__((always_inline)) { return (t_hi - j) * kBN + kBN - 1 > wrow0 + 32 * h; };
  QOp ka[kKOps];
  bf16x8 va[8], pf[2][2];
  f32x16 s[2];
  // this lane's K' operands of the tile in stage stg
  auto kops = [&](int stg) __attribute__((always_inline)) {
    const lds_u8* kt = smem + stg * kKTile;
    if constexpr (FP8) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        ka[m] = join_i32x8(__builtin_bit_cast(u32x4, lds_read_b128(kt + (kread_off ^ ((2u * m) << 4)))),
                           __builtin_bit_cast(u32x4, lds_read_b128(kt + (kread_off ^ ((2u * m + 1) << 4)))));
    } else {
      load_kops(ka, kt, kread_off);
    }
  };
  if (exact_max) {
    float mx[2] = {-INFINITY, -INFINITY};
    int stg = 0;
    for (int j = 0; j < nt; ++j) {
      // tile j has landed (the first NS before the loop; later tiles j + 1 ..
      // j + NS - 1 may fly)
      if (j > 0) sync_tiles<kCopies * (NS - 1)>();
      kops(stg);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (FP8) qk_fp8(s[h], ka, qf[h]);
        else qk_mfma(s[h], ka, qf[h]);
      }
      lds_barrier();  // every wave has read stage stg
      gload_j(j + NS, stg);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (masked(j, h)) mask_causal(s[h], qm[h] - (t_hi - j) * kBN - 4 * half);
        mx[h] = fmaxf(mx[h], blk_max(s[h]));
      }
      stg = stg + 1 == NS ? 0 : stg + 1;
    }
    sync_tiles<0>();
    fill_ring();
    sync_tiles<0>();
#pragma unroll
    for (int h = 0; h < 2; ++h) st[h].m_run = FP8 ? mx[h] * fsc[h] : mx[h];
  }
  // m_run: the row's softmax offset (exp2 units); the score accumulators
  // start from its negative (E4M3: the softmax's FMA subtracts it)
  f32x16 seed[2];
  float nu[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    nu[h] = -st[h].m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) seed[h][r] = -st[h].m_run;
  }
  // the exp2 argument of score r of half h
  auto arg = [&](int h, int r) __attribute__((always_inline)) {
    return FP8 ? __builtin_fmaf(s[h][r], fsc[h], nu[h]) : s[h][r];
  };
  auto qk = [&](int h) __attribute__((always_inline)) {
    if constexpr (FP8) qk_fp8(s[h], ka, qf[h]);
    else qk_seeded(s[h], ka, qf[h], seed[h]);
  };

  auto vops = [&](int stg) __attribute__((always_inline)) {
    const lds_u8* vr[4];
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) vr[bd] = vread0[bd] + stg * kTileBytes;
    load_vops(va, vr);
  };
  auto mask = [&](int h, int j) __attribute__((always_inline)) {
    if (masked(j, h)) mask_causal(s[h], qm[h] - (t_hi - j) * kBN - 4 * half);
  };
  // Half h's P, packed to bf16, and its row sums.  The results are consumed
  // by an empty asm at the end of the slot, so that the compiler keeps this
  // VALU work beside that slot's MFMAs instead of sinking it to the first use.
  auto softmax = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 u;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        u[w] = p_word(arg(h, 8 * t + 2 * w), arg(h, 8 * t + 2 * w + 1), st[h].l_run);
      pf[h][t] = __builtin_bit_cast(bf16x8, u);
    }
    pin(pf[h][0]);
    pin(pf[h][1]);
    pin(st[h].l_run);
  };
  // The PV MFMAs of half 1 beside half 0's P.  The scheduler cannot see the
  // asm MFMAs' latency, so the order is fixed here, software-pipelined over
  // the eight words of P: MFMA g goes with the exps of word g and the
  // packing and row sum of word g - 1, so that no step waits on the one just
  // before it and no two MFMAs are issued back to back.
  auto pv1_sm0 = [&]() __attribute__((always_inline)) {
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float e[16];
    u32x4 u[2];
    auto word = [&](int w) __attribute__((always_inline)) {
      // (bit-cast a scalar: a bit-cast of a vector element reads element 0)
      const uint32_t uw = pack_bf16x2(e[2 * w], e[2 * w + 1]);
      u[w / 4][w % 4] = uw;
      st[0].l_run =
          __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, uw), one2, st[0].l_run, false);
    };
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      pv_agpr_one(st[1].acc, va, pf[1], g);
      e[2 * g] = fast_exp2(arg(0, 2 * g));
      e[2 * g + 1] = fast_exp2(arg(0, 2 * g + 1));
      if (g > 0) word(g - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    word(7);
    pf[0][0] = __builtin_bit_cast(bf16x8, u[0]);
    pf[0][1] = __builtin_bit_cast(bf16x8, u[1]);
    pin(pf[0][0]);
    pin(pf[0][1]);
    pin(st[0].l_run);
  };

  // Per 32-key tile j the wave runs four slots; the MFMAs of each slot do not
  // depend on the VALU work beside them:
  //   A(j): S0 = K'(j+1) Q0'^T   | half 1's P of tile j
  //   B(j): O1 += V(j) P1(j)     | half 0's P of tile j + 1
  //   C(j): S1 = K'(j+1) Q1'^T   | the V(j+1) operand reads
  //   D(j): O0 += V(j+1) P0(j+1) | the K'(j+2) operand reads
  // The causal mask (only the first tiles of a wave need it) is applied
  // under a wave-uniform branch at the slot boundary before a half's P, so
  // that the slots themselves stay single blocks.

  // ---- warm-up: both halves' scores of tile 0, half 0's P and PV
  kops(0);
  qk(0);
  qk(1);
  mask(0, 0);
  softmax(0);
  vops(0);
  kops(1 % NS);  // tile 1 (or a copy of tile 0)
  lds_barrier();                          // every wave has read tile 0
  gload_j(NS, 0);
  pv_agpr(st[0].acc, va, pf[0]);

  // ---- main loop.  On entry to iteration j: S1 of tile j, ka = K'(j + 1),
  // va = V(j), O0 through tile j, O1 through tile j - 1.
  int sa = 1 % NS;  // stage of tile j + 1
  for (int j = 0; j + 1 < nt; ++j) {
    const int sb = sa + 1 == NS ? 0 : sa + 1;  // stage of tile j + 2
    mask(1, j);
    // A
    __builtin_amdgcn_sched_barrier(0);
    qk(0);
    softmax(1);
    if constexpr (!FP8) {
      // each score MFMA followed by six of the softmax's VALU instructions
      // (left to the scheduler, it clustered them: 1.1-1.3% slower at 16K
      // and 256K)
#pragma unroll
      for (int gg = 0; gg < kQkMfma; ++gg) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mask(0, j + 1);
    // B
    __builtin_amdgcn_sched_barrier(0);
    pv1_sm0();
    __builtin_amdgcn_sched_barrier(0);
    // C
    qk(1);
    vops(sa);
    // one score MFMA, then its share of the sixteen V reads (so that the
    // reads spread under the products instead of queueing at the barrier)
    if constexpr (ILV > 0) {
      static_assert(kQkMfma % ILV == 0, "whole groups of score MFMAs");
#pragma unroll
      for (int gg = 0; gg < kQkMfma / ILV; ++gg) {
        __builtin_amdgcn_sched_group_barrier(0x008, ILV, 0);   // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 16 * ILV / kQkMfma, 0);  // LDS reads
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // tile j + 2 has landed for every wave, and no wave still reads tile
    // j + 1's stage, which takes tile j + 1 + NS
    sync_tiles<kCopies * (NS - 2)>();
    gload_j(j + 1 + NS, sa);
    // D
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FP8) {
      pv_agpr(st[0].acc, va, pf[0]);
      kops(sb);
    } else {
      // each PV MFMA followed by one of the next tile's K' operand reads, in
      // this order (left to the scheduler: 1.1% slower at 16K, 1.5% at 256K)
      const lds_u8* kt = smem + sb * kKTile;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv_agpr_one(st[0].acc, va, pf[0], i);
        ka[i] = lds_read_b128(kt + (kread_off ^ (uint32_t)(i << 4)));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    sa = sb;
  }
  int ticket = -1;
  if (wv == 0) ticket = claim_own(p.queue, own, own_done);  // read after the epilogue
  // ---- tail: half 1 of the last tile
  mask(1, nt - 1);
  softmax(1);
  pv_agpr(st[1].acc, va, pf[1]);

  // ---- epilogue: normalise, gate (if any), store.  Register r of block bd,
  // lane half h -> dim 32 bd + 8 (r/4) + 4 h + r%4: four runs of 4 dims.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    acc_settle(st[h].acc);
    const float l_tot = pair_sum32(st[h].l_run);
    const float inv = 1.0f / l_tot;
    if (p.lse && qok[h] && half == 0)
      p.lse[lse0 + head * lse_hs + qi[h]] = (st[h].m_run + __log2f(l_tot)) * kLn2;
    if (!qok[h]) continue;
    const long long qrow = (tok0 + qi[h]) * p.Hq + head;
    uint16_t* dst = p.out + qrow * kD + 4 * half;
    const uint16_t* gsrc = p.gate ? p.gate + qrow * kD + 4 * half : nullptr;
    // the gate words of the row first (all sixteen loads in flight at once)
    uint2 gg[16];
    if (gsrc) {
#pragma unroll
      for (int i = 0; i < 16; ++i) gg[i] = *reinterpret_cast<const uint2*>(gsrc + 32 * (i / 4) + 8 * (i % 4));
    }
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st[h].acc[bd][4 * q4 + e] * inv;
        const int off = 32 * bd + 8 * q4;
        if (gsrc) {
          const uint2 g2 = gg[4 * bd + q4];
          o[0] *= sigmoidf_(bf_lo(g2.x));
          o[1] *= sigmoidf_(bf_hi(g2.x));
          o[2] *= sigmoidf_(bf_lo(g2.y));
          o[3] *= sigmoidf_(bf_hi(g2.y));
        }
        uint2 w;
        w.x = pack_bf16x2(o[0], o[1]);
        w.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(dst + off) = w;
      }
    }
  }
  wait_vm<0>();  // the ring copies of tiles past the end, the stores and the claim
  // (read on every lane, so that the compiler's own wait for the claim sits
  // here on every path, not at the next job's first loads)
  const int tk = __builtin_amdgcn_readfirstlane(ticket);
  if (wv == 0) next = next_job(p.queue, own, geo.nq, geo.n_jobs, own_done, tk);
  };

  // ---- persistent loop: one workgroup per CU takes jobs until every queue
  // is empty.  The barrier at the top of each pass publishes the job and
  // ends the previous job's use of the LDS ring.  Each job ends with its
  // memory operations complete (its output stores included): letting them
  // run into the next job was 1% faster at 16K and 64K but 7-10% slower at
  // 256K, on three boxes.
  if (wv == 0)
    job_s[0] = next_job(p.queue, own, geo.nq, geo.n_jobs, own_done,
                        __builtin_amdgcn_readfirstlane(claim_own(p.queue, own, own_done)));
  for (int it = 0;; ++it) {
    __syncthreads();
    const int job = __builtin_amdgcn_readfirstlane(job_s[it & 1]);
    if (job < 0) break;
    int next = -1;
    run_job(job, next);
    if (wv == 0) job_s[(it + 1) & 1] = next;
  }
}

constexpr int kCStages = 8;

// Interleaved schedules by length: bf16 sequences longer than this use
// groups of two, shorter ones groups of one; E4M3 sequences longer than it
// are not interleaved.
constexpr int kIlvLongS = 65536;

template <int RH, bool PACKED, bool FP8 = false, int ILV = 1>
void launch_causal(dim3 grid, hipStream_t stream, const FlashParams& p, const Geo& geo) {
  hipLaunchKernelGGL((flash_causal_kernel<RH, PACKED, kCStages, FP8, ILV>), grid, dim3(kCThreads),
                     0, stream, p, geo);
}

}  // namespace

hipError_t launch_flash_causal(const FlashParams& p, hipStream_t stream) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  const int grp = p.Hq / p.Hkv;
  Geo geo;
  geo.heads_per_wg = grp < kCWaves ? grp : kCWaves;
  geo.hgroups = grp / geo.heads_per_wg;
  geo.pos_per_wg = kCRows * kCWaves / geo.heads_per_wg;
  geo.n_pos_blocks = (p.S + geo.pos_per_wg - 1) / geo.pos_per_wg;
  geo.n_bhg = p.B * p.Hkv * geo.hgroups;
  const long long blocks = (long long)geo.n_pos_blocks * geo.n_bhg;
  if (blocks > 0x3fffffffLL || !p.queue) return hipErrorInvalidValue;
  // persistent grid: one workgroup per CU (each takes a whole CU's LDS)
  geo.n_jobs = (int)blocks;
  const int wgs = (int)std::min<long long>(blocks, device_cu_count());
  geo.nq = std::min(wgs, 8);
  const dim3 grid((unsigned)wgs);
  const bool long_s = p.S > kIlvLongS;
  if (p.kp8) {  // the E4M3 variant: fixed-length batches
    if (p.cu_seqlens) return hipErrorInvalidValue;
    if (p.rope_half == 21 && long_s) launch_causal<21, false, true, 0>(grid, stream, p, geo);
    else if (p.rope_half == 21) launch_causal<21, false, true>(grid, stream, p, geo);
    else if (p.rope_half == 0) launch_causal<0, false, true>(grid, stream, p, geo);
    else launch_causal<-1, false, true>(grid, stream, p, geo);
  } else if (p.cu_seqlens) {
    if (p.rope_half == 21) launch_causal<21, true>(grid, stream, p, geo);
    else if (p.rope_half == 0) launch_causal<0, true>(grid, stream, p, geo);
    else launch_causal<-1, true>(grid, stream, p, geo);
  } else {
    if (p.rope_half == 21 && long_s) launch_causal<21, false, false, 2>(grid, stream, p, geo);
    else if (p.rope_half == 21) launch_causal<21, false>(grid, stream, p, geo);
    else if (p.rope_half == 0) launch_causal<0, false>(grid, stream, p, geo);
    else launch_causal<-1, false>(grid, stream, p, geo);
  }
  return hipGetLastError();
}

}  // namespace zg
