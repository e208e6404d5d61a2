// QK-RMSNorm + partial RoPE of the keys.
//
// Page "7B 打 235B？中关村学院把'小模型怎么活'这道题答成了一份全开源配方"
// (shibing624.github.io), section 🏗️ 架构: Q and K are normalised with
// RMSNorm and rotated with RoPE on a 0.33 fraction of the head dim.  Here, per
// key row of D = 128 values: x_hat = x / sqrt(mean(x^2) + eps) * w, then the
// first R dims are rotated pairwise (t, t + R/2) by pos * theta^(-2t/R); the
// remaining dims pass through.  The queries get the same treatment inside the
// attention kernels, fused into their Q-tile loads.
//
// Layout: 16 lanes per row, 8 bf16 (16 bytes) per lane, groups of 16 rows
// per 256-thread block (the key prologue strides a fixed grid over the
// groups; the decode append takes one group per block).  The row's
// normalised values go through LDS so that each lane can read the partner
// dim of its rotary pairs.

#include "zg_common.h"
#include "zg_fp8.h"
#include "zg_launch.h"
#include "zg_norm_rope.h"

namespace zg {

namespace {

constexpr int kRowsPerBlock = 16;
constexpr long long kPrologueBlocks = 2048;

// kout receives K' * k_scale: as bf16 (the product in fp32, rounded once), or
// with FP8 as E4M3 codes (one byte per element).
template <bool FP8>
__global__ __launch_bounds__(256) void k_prologue_kernel(const uint16_t* __restrict__ k,
                                                         const float* __restrict__ w,
                                                         void* __restrict__ kout,
                                                         long long rows, int S, int Hkv,
                                                         const int* __restrict__ cu_seqlens,
                                                         int nseq, long long pos_offset,
                                                         int rope_half, float eps, RopeTable tab,
                                                         float k_scale, int* zero16) {
  // the causal kernel's work-queue counters, cleared for the launch after
  if (zero16 && blockIdx.x == 0 && threadIdx.x < 16) zero16[threadIdx.x] = 0;
  __shared__ float xs[kRowsPerBlock][kD];
  __shared__ float cs[kRowsPerBlock][kMaxRopeHalf], sn[kRowsPerBlock][kMaxRopeHalf];
  const int lrow = threadIdx.x / 16;
  const int c16 = threadIdx.x % 16;
  // Groups of 16 rows, strided over a fixed grid; each group's rows are
  // loaded two groups ahead (the loop is unrolled by two, so each of the two
  // buffers is refilled in place as soon as it is consumed).  Rows past the
  // end read row rows - 1 (in bounds, no branch) and store nothing.
  auto load = [&](long long rg) {
    return ld16(k + min(rg * kRowsPerBlock + lrow, rows - 1) * kD + 8 * c16);
  };
  const RowConsts kc = row_consts(w, rope_half, tab, c16);
  const long long G = gridDim.x;
  auto body = [&](long long rg, u32x4& xu) __attribute__((always_inline)) {
    const long long row = rg * kRowsPerBlock + lrow;
    const bool ok = row < rows;
    float x[8];
    unpack_bf16x8(xu, x);
    xu = load(rg + 2 * G);
    // position of the row's token within its sequence
    const long long tok = row / Hkv;
    long long s;
    if (cu_seqlens) {  // packed: the last sequence b with cu_seqlens[b] <= tok
      int lo = 0, hi = nseq;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_seqlens[mid] <= tok) lo = mid;
        else hi = mid;
      }
      s = max(tok - (long long)cu_seqlens[lo], 0LL);
    } else {
      s = tok % S;
    }
    // rows are (b, s, head): the first row of each position in the group
    // computes the angles for all of them
    const int hh = (int)(row % Hkv);
    const int ref = lrow - min(hh, lrow);
    norm_rope_row(x, c16, kc, eps, rope_half, pos_offset + s, xs[lrow], ref == lrow, cs[lrow],
                  sn[lrow], cs[ref], sn[ref]);
    if (ok) {
      if constexpr (FP8) {
        st8(static_cast<uint8_t*>(kout) + row * kD + 8 * c16, pack_e4m3x8(x, k_scale));
      } else {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i] * k_scale, x[2 * i + 1] * k_scale);
        st16(static_cast<uint16_t*>(kout) + row * kD + 8 * c16, o);
      }
    }
    lds_barrier();  // xs and the angle tables are rewritten by the next group
  };
  u32x4 xa = load(blockIdx.x);
  u32x4 xb = load(blockIdx.x + G);
  for (long long rg = blockIdx.x; rg * kRowsPerBlock < rows; rg += 2 * G) {  // uniform
    body(rg, xa);
    if ((rg + G) * kRowsPerBlock < rows) body(rg + G, xb);
  }
}

// Decode: normalise + rotate the new key of each (b, kv head) at position
// pos_offset + len - 1 and write it, with the new value, into its cache slot.
// FP8: the caches hold E4M3 codes of K' * k_scale and V * v_scale (one byte
// per element, same layout).
template <bool FP8>
__global__ __launch_bounds__(256) void decode_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    void* __restrict__ k_cache, void* __restrict__ v_cache,
    const int* __restrict__ seq_lens, const float* __restrict__ w, int rows, int Hkv,
    int cap, int ring, CacheMap map, long long pos_offset, int rope_half, float eps,
    RopeTable tab, float k_scale, float v_scale) {
  __shared__ float xs[kRowsPerBlock][kD];
  __shared__ float cs[kRowsPerBlock][kMaxRopeHalf], sn[kRowsPerBlock][kMaxRopeHalf];
  const int lrow = threadIdx.x / 16;
  const int c16 = threadIdx.x % 16;
  const int row = blockIdx.x * kRowsPerBlock + lrow;  // b * Hkv + g
  const bool ok = row < rows;
  const int b = ok ? row / Hkv : 0;
  int L = ok ? seq_lens[b] : 1;
  L = L < 1 ? 1 : L;
  if (!ring && L > cap) L = cap;
  const int slot = ring ? (L - 1) % cap : L - 1;
  float x[8];
  u32x4 vv = {0, 0, 0, 0};
  if (ok) {
    unpack_bf16x8(ld16(k_new + (long long)row * kD + 8 * c16), x);
    vv = ld16(v_new + (long long)row * kD + 8 * c16);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  // rows are (b, kv head): one position per b
  const int ref = lrow - min(row % Hkv, lrow);
  norm_rope_row(x, c16, w, eps, rope_half, tab, pos_offset + L - 1, xs[lrow], ref == lrow,
                cs[lrow], sn[lrow], cs[ref], sn[ref]);
  if (ok) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    long long dst;
    if (map.block_table) {  // slot L-1 of its page
      const int pg = map.page(b, slot);
      dst = ((((long long)pg * Hkv + row % Hkv) << map.page_shift) + (slot & ((1 << map.page_shift) - 1))) * kD + 8 * c16;
    } else {
      dst = ((long long)row * cap + slot) * kD + 8 * c16;
    }
    if constexpr (FP8) {
      float vf[8];
      unpack_bf16x8(vv, vf);
      st8(static_cast<uint8_t*>(k_cache) + dst, pack_e4m3x8(x, k_scale));
      st8(static_cast<uint8_t*>(v_cache) + dst, pack_e4m3x8(vf, v_scale));
    } else {
      st16(static_cast<uint16_t*>(k_cache) + dst, o);
      st16(static_cast<uint16_t*>(v_cache) + dst, vv);
    }
  }
}

// Prefill -> paged cache: token s of sequence b (rows of [B,S,Hkv,D]) goes
// to slot s % page_size of page block_table[b][s / page_size].  16 lanes per
// row, 16 bytes each.
__global__ __launch_bounds__(256) void kv_write_pages_kernel(const uint16_t* __restrict__ kp,
                                                             const uint16_t* __restrict__ v,
                                                             uint16_t* __restrict__ k_pages,
                                                             uint16_t* __restrict__ v_pages,
                                                             long long rows, int S, int Hkv,
                                                             CacheMap map) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b*S + s)*Hkv + g
  const int c16 = threadIdx.x & 15;
  if (row >= rows) return;
  const int g = (int)(row % Hkv);
  const long long bs = row / Hkv;
  const int s = (int)(bs % S);
  const long long b = bs / S;
  const int pg = map.page(b, s);
  const long long dst =
      ((((long long)pg * Hkv + g) << map.page_shift) + (s & ((1 << map.page_shift) - 1))) * kD + 8 * c16;
  st16(k_pages + dst, ld16(kp + row * kD + 8 * c16));
  st16(v_pages + dst, ld16(v + row * kD + 8 * c16));
}

}  // namespace

static long long prologue_blocks(long long rows) {
  // eight 256-thread blocks per CU stride over the groups of 16 rows
  const long long groups = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  return groups < kPrologueBlocks ? groups : kPrologueBlocks;
}

hipError_t launch_k_prologue(const uint16_t* k, const float* w, uint16_t* kout, long long rows,
                             int S, int Hkv, long long pos_offset, int rope_half, float eps,
                             const RopeTable& tab, hipStream_t stream, const int* cu_seqlens,
                             int nseq, float out_scale, int* zero16) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prologue_kernel<false>, dim3((unsigned)prologue_blocks(rows)), dim3(256), 0,
                     stream, k, w, (void*)kout, rows, S, Hkv, cu_seqlens, nseq, pos_offset,
                     rope_half, eps, tab, out_scale, zero16);
  return hipGetLastError();
}

hipError_t launch_k_prologue_fp8(const uint16_t* k, const float* w, uint8_t* kout, float k_scale,
                                 long long rows, int S, int Hkv, long long pos_offset,
                                 int rope_half, float eps, const RopeTable& tab,
                                 hipStream_t stream, const int* cu_seqlens, int nseq,
                                 int* zero16) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prologue_kernel<true>, dim3((unsigned)prologue_blocks(rows)), dim3(256), 0,
                     stream, k, w, (void*)kout, rows, S, Hkv, cu_seqlens, nseq, pos_offset,
                     rope_half, eps, tab, k_scale, zero16);
  return hipGetLastError();
}

hipError_t launch_decode_append(const uint16_t* k_new, const uint16_t* v_new, void* k_cache,
                                void* v_cache, const int* seq_lens, const float* w, int B,
                                int Hkv, int cap, int ring, const CacheMap& map,
                                long long pos_offset, int rope_half, float eps,
                                const RopeTable& tab, int fp8, float k_scale, float v_scale,
                                hipStream_t stream) {
  const int rows = B * Hkv;
  if (rows == 0) return hipSuccess;
  const int blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (fp8)
    hipLaunchKernelGGL(decode_append_kernel<true>, dim3(blocks), dim3(256), 0, stream, k_new,
                       v_new, k_cache, v_cache, seq_lens, w, rows, Hkv, cap, ring, map,
                       pos_offset, rope_half, eps, tab, k_scale, v_scale);
  else
    hipLaunchKernelGGL(decode_append_kernel<false>, dim3(blocks), dim3(256), 0, stream, k_new,
                       v_new, k_cache, v_cache, seq_lens, w, rows, Hkv, cap, ring, map,
                       pos_offset, rope_half, eps, tab, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_write_pages(const uint16_t* kp, const uint16_t* v, uint16_t* k_pages,
                                 uint16_t* v_pages, int B, int S, int Hkv, const CacheMap& map,
                                 hipStream_t stream) {
  const long long rows = (long long)B * S * Hkv;
  if (rows == 0) return hipSuccess;
  const long long blocks = (rows + 15) / 16;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_write_pages_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kp, v,
                     k_pages, v_pages, rows, S, Hkv, map);
  return hipGetLastError();
}

}  // namespace zg
