// The projections on either side of the attention: y = x W^T with bf16
// operands, fp32 accumulation on MFMA and bf16 results.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 核心方法, and page "7B 打 235B？中关村学院把'小模型怎么活'这道题答成了
// 一份全开源配方" (shibing624.github.io), section 🏗️ 架构: hidden size 4096,
// 32 query and 8 KV heads of 128 dims, and a sigmoid gate of the output's
// shape on the sliding-window layers.  The input projection of a layer is one
// GEMM against the stacked weight [W_q; W_k; W_v; W_g] (10240 x 4096 on a
// gated layer) whose epilogue writes q, k, v and the gate logits straight
// into the four token-major tensors the attention kernels read; the output
// projection is the same kernel with one output.
//
// Both operands are K-contiguous ("TN"): x is [M, K] and W is [N, K], row
// major, which is exactly the per-lane layout of both MFMA operands (8
// consecutive k of one row per lane).
//
// Workgroup tile 256 x 256, eight waves in a 2 (M) x 4 (N) grid, each wave
// 128 x 64 = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16, 128 KB of LDS.  Tiles
// move global -> LDS with untracked global_load_lds_dwordx4 copies.  Two
// instances: K step 64 (128-byte LDS rows, eight 16-byte chunks XOR-swizzled
// by (row / 2) % 8, a two-stage ring whose next step's copies fly during the
// current step's MFMAs) when K is a multiple of 64, else K step 32 (64-byte
// rows, four chunks swizzled by (row / 4) % 4, a four-stage ring filled three
// steps ahead).  Both swizzles make every MFMA operand read conflict-free
// under the 64-bank LDS.  The FP8 instance takes E4M3 operands at K step 128
// (128-byte rows) on v_mfma_scale_f32_32x32x64_f8f6f4.

#include "zg_common.h"
#include "zg_fp8.h"
#include "zg_launch.h"
#include "zg_lds.h"

namespace zg {

namespace {

constexpr int kGBM = 256, kGBN = 256;

// LDS rows of ROWB bytes (64 or 128) per K step: a K step is ROWB / 2
// bf16 or ROWB fp8 elements.  Rows of A then W per stage; a 1 KB copy covers
// 1024 / ROWB rows.
template <int ROWB, int W> struct GCfg {
  static constexpr int kRowBytes = ROWB;
  static constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per row
  static constexpr int kStages = ROWB == 64 ? 4 : 2;
  static constexpr int kTileA = kGBM * kRowBytes;
  static constexpr int kTileB = kGBN * kRowBytes;
  static constexpr int kStageBytes = kTileA + kTileB;
  static constexpr int kSmem = kStages * kStageBytes;     // 131072
  static constexpr int kBlocksPerWave = kTileA / 1024 / W;  // per operand
  static constexpr int kCopies = 2 * kBlocksPerWave;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  // chunk swizzle: rows that share a 256-byte bank window, and successive
  // windows, get distinct chunk positions
  __device__ static int swz(int row) {
    return ROWB == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
  }
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The MFMA of each element type: bf16 v_mfma_f32_32x32x16_bf16 (16 k per
// instruction, 16 bytes per lane) or FP8 E4M3 v_mfma_scale_f32_32x32x64_f8f6f4
// (64 k, 32 bytes per lane: row l % 32, k 32 (l / 32) + 4 d + byte j of dword
// d, probe-confirmed; block scales fixed at 1).  CPL: 16-byte chunks per lane
// per instruction.
template <bool FP8> struct GOp;
template <> struct GOp<false> {
  typedef bf16x8 T;
  static constexpr int CPL = 1;
  __device__ static T read(const lds_u8* st, const uint32_t (&a)[1]) { return lds_read_b128(st + a[0]); }
  __device__ static f32x16 mma(const T& a, const T& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct GOp<true> {
  typedef i32x8 T;
  static constexpr int CPL = 2;
  __device__ static T read(const lds_u8* st, const uint32_t (&a)[2]) {
    const u32x4 lo = __builtin_bit_cast(u32x4, lds_read_b128(st + a[0]));
    const u32x4 hi = __builtin_bit_cast(u32x4, lds_read_b128(st + a[1]));
    return T{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  __device__ static f32x16 mma(const T& a, const T& b, const f32x16& c) {
    // formats 0 / 0: E4M3 for A and B; E8M0 block scales 127 = 1.0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// W waves in a 2 (M) x W/2 (N) grid: a wave computes 128 x 512/W, i.e.
// 4 x NB blocks of 32 x 32 (W = 8: two waves per SIMD, 128 accumulator
// registers each; W = 4: one wave per SIMD, 256, which the compiler may keep
// in the accumulation registers).
template <int ROWB, int W, bool FP8>
__global__ __launch_bounds__(64 * W, 1) void gemm_bf16_tn_kernel(GemmParams p) {
  using C = GCfg<ROWB, W>;
  using O = GOp<FP8>;
  using OT = typename O::T;
  constexpr int EB = FP8 ? 1 : 2;  // bytes per element
  constexpr int NB = 16 / W;  // 32-column blocks per wave: 256 / (W / 2) columns
  static_assert(NB * 32 * (W / 2) == kGBN && 4 * 32 * 2 == kGBM, "waves must tile 256 x 256");
  constexpr int kGStages = C::kStages;
  constexpr int kGStageBytes = C::kStageBytes;
  constexpr int kGTileA = C::kTileA;
  constexpr int kGRowBytes = C::kRowBytes;
  constexpr int kGCopies = C::kCopies;
  constexpr int BPW = C::kBlocksPerWave;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[C::kSmem];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int wm = wvu & 1;   // M half of the tile
  const int wn = wvu >> 1;  // N quarter of the tile

  // ---- tile of this workgroup.  Consecutive workgroup ids go to different
  // XCDs; each XCD is given a contiguous range of tiles, walked in groups of
  // kGroupM tile rows so that the workgroups resident on one XCD share A
  // panels and W panels in its L2.
  const int ntiles = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  int lin = bid;
  if (ntiles % 8 == 0) lin = (bid % 8) * (ntiles / 8) + bid / 8;
  constexpr int kGroupM = 4;
  const int per_group = kGroupM * p.tiles_n;
  const int grp = lin / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(p.tiles_m - first_m, kGroupM);
  const int tm = first_m + (lin % per_group) % gsize;
  const int tn = (lin % per_group) / gsize;
  const int m0 = tm * kGBM;
  const int n0 = tn * kGBN;

  // ---- copies: block j of this wave covers rows R (BPW wv + j) .. +R-1 of
  // the A (resp. W) tile (R rows per 1 KB); lane L writes physical chunk
  // L % chunks of row L / chunks of the block and fetches the logical chunk
  // stored there.
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(p.a) +
                               (long long)m0 * p.lda * EB;
  const unsigned char* bbase = reinterpret_cast<const unsigned char*>(p.b) +
                               (long long)n0 * p.ldb * EB;
  uint32_t aoff[BPW], boff[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int row = C::kRowsPerCopy * (BPW * wvu + j) + lane / C::kChunks;
    const int lc = (lane % C::kChunks) ^ C::swz(row);
    const int arow = min(row, p.M - 1 - m0);  // rows past M repeat row M-1
    aoff[j] = (uint32_t)(arow * p.lda * EB + lc * 16);
    boff[j] = (uint32_t)(row * p.ldb * EB + lc * 16);
  }
  auto issue = [&](int ks, int stg) {
    const unsigned char* ak = abase + (long long)ks * ROWB;
    const unsigned char* bk = bbase + (long long)ks * ROWB;
    const uint32_t la = lds_addr(smem + stg * kGStageBytes) + (BPW * wvu) * 1024;
    const uint32_t lb = la + kGTileA;
#pragma unroll
    for (int j = 0; j < BPW; ++j) dma16_s(ak, aoff[j], la + j * 1024);
#pragma unroll
    for (int j = 0; j < BPW; ++j) dma16_s(bk, boff[j], lb + j * 1024);
  };

  // ---- operand reads: lane l reads row l % 32 of a 32-row block, logical
  // chunks 2 CPL kk + CPL (l / 32) + c (kk: the slices of the K step that
  // one MFMA consumes)
  const int r32 = lane & 31;
  const int hsel = lane >> 5;
  constexpr int CPL = O::CPL;
  constexpr int KK = C::kChunks / (2 * CPL);
  uint32_t ard[4][KK][CPL], brd[NB][KK][CPL];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int row = wm * 128 + mb * 32 + r32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        ard[mb][kk][c] = row * kGRowBytes + (((2 * CPL * kk + CPL * hsel + c) ^ C::swz(row)) << 4);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = wn * 32 * NB + nb * 32 + r32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        brd[nb][kk][c] = kGTileA + row * kGRowBytes + (((2 * CPL * kk + CPL * hsel + c) ^ C::swz(row)) << 4);
  }

  f32x16 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

  const int nk = p.K / (ROWB / EB);
  auto mfmas = [&](const OT (&af)[4], const OT (&bfr)[NB]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = O::mma(af[mb], bfr[nb], acc[mb][nb]);
  };
  auto load_ops = [&](OT (&af)[4], OT (&bfr)[NB], const lds_u8* st, int kk) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[mb] = O::read(st, ard[mb][kk]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) bfr[nb] = O::read(st, brd[nb][kk]);
  };

  if constexpr (kGStages == 2 && !FP8) {
    // Two stages, software-pipelined: the operands of slice kk+1 are read
    // while the MFMAs of slice kk run, also across steps.  At the last
    // slice of step ks every wave has issued (and, at the barrier, received)
    // all its reads of step ks, and step ks+1 has landed: after the barrier
    // the copies of step ks+2 refill stage ks % 2 and slice 0 of step ks+1 is
    // read, under the last MFMAs of step ks.
    static_assert(KK % 2 == 0, "operand buffers alternate per slice");
    OT af[2][4], bfr[2][NB];
    issue(0, 0);
    if (nk > 1) issue(1, 1);
    if (nk > 1) sync_tiles<kGCopies>();
    else sync_tiles<0>();
    load_ops(af[0], bfr[0], smem, 0);
    for (int ks = 0; ks < nk; ++ks) {
      const lds_u8* st = smem + (ks & 1) * kGStageBytes;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        if (kk + 1 < KK) {
          load_ops(af[nxt], bfr[nxt], st, kk + 1);
        } else if (ks + 1 < nk) {
          sync_tiles<0>();
          if (ks + 2 < nk) issue(ks + 2, ks & 1);
          load_ops(af[nxt], bfr[nxt], smem + ((ks + 1) & 1) * kGStageBytes, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas(af[cur], bfr[cur]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < kGStages - 1; ++s)
      if (s < nk) issue(s, s);

    // (FP8 takes this loop with two stages: its operands are twice the
    // registers of bf16's, too many to double-buffer)
    for (int ks = 0; ks < nk; ++ks) {
      // step ks has landed for every wave; the groups of the following
      // steps (up to kGStages - 2 of them) may still fly.  Every wave's reads
      // of step ks-1 are done (lgkmcnt(0)), so its stage can be refilled.
      if (kGStages >= 4 && ks + 2 < nk) sync_tiles<2 * kGCopies>();
      else if (kGStages >= 3 && ks + 1 < nk) sync_tiles<kGCopies>();
      else sync_tiles<0>();
      if (ks + kGStages - 1 < nk) issue(ks + kGStages - 1, (ks + kGStages - 1) % kGStages);
      const lds_u8* st = smem + (ks % kGStages) * kGStageBytes;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        OT af[4], bfr[NB];
        load_ops(af, bfr, st, kk);
        mfmas(af, bfr);
      }
    }
  }

  // ---- epilogue: the N tile lies in one output segment; register r of
  // block (mb, nb) holds row 8 (r/4) + 4 (l/32) + r%4, column l % 32
  int sg = 0;
#pragma unroll
  for (int i = 1; i < kGemmMaxSegs; ++i)
    if (i < p.nseg && n0 >= p.seg[i].n0) sg = i;
  uint16_t* out = p.seg[sg].ptr;
  const long long ld = p.seg[sg].ld;
  const int ncol0 = n0 - p.seg[sg].n0 + wn * 32 * NB + r32;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3);
      if (row < p.M) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          out[row * ld + ncol0 + nb * 32] =
              __builtin_bit_cast(uint16_t, (__bf16)(FP8 ? acc[mb][nb][r] * p.out_scale : acc[mb][nb][r]));
      }
    }
  }
}

constexpr int kGemmWaves = 8;

// bf16 -> FP8 E4M3: q = RNE(clamp(x * scale, -448, 448)), the product taken
// in fp32.  The conversion instruction does not saturate (its overflow is
// NaN), hence the explicit clamp.  8 elements per lane.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ q, long long n8,
                                                           float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  unpack_bf16x8(ld16(x + 8 * i), v);
  st8(q + 8 * i, pack_e4m3x8(v, scale));
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* x, uint8_t* q, long long n, float scale,
                               hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const long long n8 = n / 8;
  const long long blocks = (n8 + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, n8,
                     scale);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_tn(GemmParams p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  if (p.N % kGBN || p.K % (p.fp8 ? 128 : 32) || p.K < 32 || p.nseg < 1 || p.nseg > kGemmMaxSegs)
    return hipErrorInvalidValue;
  p.tiles_m = (p.M + kGBM - 1) / kGBM;
  p.tiles_n = p.N / kGBN;
  const long long blocks = (long long)p.tiles_m * p.tiles_n;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr int W = kGemmWaves;
  const dim3 grid((unsigned)blocks), block(64 * W);
  if (p.fp8)
    hipLaunchKernelGGL((gemm_bf16_tn_kernel<128, W, true>), grid, block, 0, stream, p);
  else if (p.K % 64 == 0)
    hipLaunchKernelGGL((gemm_bf16_tn_kernel<128, W, false>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_bf16_tn_kernel<64, W, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace zg
