// Split-KV decode attention and its log-sum-exp merge.
//
// Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
// section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: the sliding-window
// layers keep a constant-size KV cache (here a ring of `window` slots); the
// global layers keep every position.  Structured-data table, row
// "256K 上下文推理 KV 缓存": at 256K tokens the cache of the 5 global layers is
// what decode must stream.  Page "7B 打 235B？…全开源配方", section 🏗️ 架构:
// the sliding-window output is multiplied by a sigmoid gate.
//
// One new query token per sequence.  A 256-thread workgroup takes one
// (batch, kv head, split) and the query heads of that kv head (the GQA group,
// up to 8, padded to the 16 columns of v_mfma_f32_16x16x32_bf16).  Its four
// waves stream disjoint 32-key slices of the split's key range straight from
// HBM (16-byte loads): S^T = K' Q'^T on MFMA, online softmax in fp32, then
// O^T += V^T P^T with the V slice transposed through a wave-private LDS tile.
// Each workgroup writes an unnormalised partial (max, sum, acc[128]) per query
// head; the merge kernel combines the splits and applies the gate.
//
// The cache is either one contiguous [cap, 128] slab per (b, kv head) or a
// pool of fixed-size pages addressed through a per-sequence page table (the
// PAGED instance); both read the same keys in the same order, so they give
// the same bits.  It holds bf16 values or, in the FP8 instance, E4M3 codes
// with per-tensor scales, which halves the bytes a step streams (page
// "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 前置知识 › FP8
// 混合精度训练与 TWEO: the model's E4M3 format and per-tensor scaling).

#include "zg_common.h"
#include "zg_fp8.h"
#include "zg_launch.h"
#include "zg_norm_rope.h"

namespace zg {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerIter = kKeysPerWave * kWaves;
constexpr int kVtwStride = kKeysPerWave + 8;  // bf16 per V^T row of a wave tile (80 B)
constexpr int kQsStride = kD + 8;             // bf16 per Q' operand row (272 B)
constexpr int kMaxGroup = 8;
constexpr float kRescaleThreshold = 8.0f;

// LDS carve-up (bytes)
constexpr int kVtBytes = kWaves * kD * kVtwStride * 2;        // 40960, reused for the reduction
constexpr int kQsBytes = 16 * kQsStride * 2;                  // 4352
constexpr int kQnBytes = kMaxGroup * kD * 4;                  // 4096
constexpr int kRedOBytes = kWaves * kMaxGroup * kD * 4;       // 16384 (inside the Vt area)
static_assert(kRedOBytes <= kVtBytes, "reduction area must fit in the V^T area");
static_assert(16 * (kD + 2 * kMaxRopeHalf) * 4 <= kVtBytes, "append scratch must fit in the V^T area");

// Device-coherent fp32 store and load (agent-scope atomics: write-through,
// and a read of the coherent copy), for data that one workgroup of a launch
// hands to another.
__device__ __forceinline__ void store_coherent(float* q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup's shared memory (one instance per kernel).
struct DecodeLds {
  __attribute__((aligned(16))) unsigned char smem[kVtBytes + kQsBytes + kQnBytes];
  float red_m[kWaves][16];
  float red_l[kWaves][16];
  int last;
};

// FUSED: the launch has one split per (b, kv head), so this workgroup owns
// the whole key range: it appends the new token itself, before reading the
// cache, and writes the normalised, gated output instead of a partial.
// BLOCK: the workgroup belongs to a launch that decodes a whole block of
// layers (decode_block_kernel).  A layer with several splits then needs no
// other launch: the split whose key range holds the new token's slot appends
// the token before reading the cache, and the last split of each (b, kv
// head) to finish merges all of its splits' partials (a ticket counter per
// (b, kv head), left at zero again for the next step).
// FP8: the cache holds E4M3 codes (one byte per element).  S^T = K' Q'^T
// runs on the FP8 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4): the key
// codes as loaded (32 consecutive bytes of a key row per lane) against the
// query rows quantized per head with a power-of-two scale.  The value codes
// are widened to bf16 in registers, which is exact, for the bf16 PV MFMAs.
// The launch folds 1 / k_scale into the score scale, each lane multiplies in
// its head's 1 / s_q, and the epilogue multiplies by 1 / v_scale.
template <bool PAGED, bool FUSED, bool FP8, bool BLOCK>
__device__ __forceinline__ void decode_split_body(const DecodeParams& p, int bid, DecodeLds& lds) {
  unsigned char* smem = lds.smem;
  auto& red_m = lds.red_m;
  auto& red_l = lds.red_l;
  uint16_t* vt_all = reinterpret_cast<uint16_t*>(smem);
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + kVtBytes);
  float* qn = reinterpret_cast<float*>(smem + kVtBytes + kQsBytes);
  float* red_o = reinterpret_cast<float*>(smem);  // after the key loop

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int col = lane & 15;  // MFMA column: query head within the group
  const int kg = lane >> 4;   // 0..3
  const int grp = p.Hq / p.Hkv;

  const int split = bid % p.nsplit;
  const int bg = bid / p.nsplit;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  int L = p.seq_lens[b];
  L = L < 1 ? 1 : L;
  if (!p.ring && L > p.cap) L = p.cap;
  const int W = p.ring ? p.cap : p.window;
  const int lo = p.ring ? 0 : (W > 0 ? max(0, L - W) : 0);
  const int hi = p.ring ? min(L, p.cap) : L;
  const int n = hi - lo;
  const int chunk = (((n + p.nsplit - 1) / p.nsplit) + 63) & ~63;
  const int start = min(hi, lo + split * chunk);
  const int end = min(hi, start + chunk);

  const long long pos = p.pos_offset + L - 1;
  const int psh = p.map.page_shift;
  // raw query rows c = wv, wv + 4 of the group (loaded up front: their
  // latency overlaps the append) and, for the single-split epilogue, the gate
  // values of this thread's output elements
  float xq[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wv + kWaves * j;
    const uint16_t* src = p.q + ((long long)b * p.Hq + g * grp + min(c, grp - 1)) * kD;
    xq[j][0] = __uint_as_float((uint32_t)src[lane] << 16);
    xq[j][1] = __uint_as_float((uint32_t)src[64 + lane] << 16);
  }
  float gpre[kMaxGroup * kD / kThreads];
  if constexpr (FUSED) {
#pragma unroll
    for (int j = 0; j < kMaxGroup * kD / kThreads; ++j) {
      const int idx = tid + j * kThreads;
      gpre[j] = 0.f;
      if (p.gate && idx < grp * kD)
        gpre[j] = __uint_as_float(
            (uint32_t)p.gate[((long long)b * p.Hq + g * grp) * kD + idx] << 16);
    }
  }
  // the workgroup that appends the new token (workgroup-uniform)
  bool append = false;
  if constexpr (FUSED) {
    append = p.k_new != nullptr;
  } else if constexpr (BLOCK) {
    const int slot_new = p.ring ? (L - 1) % p.cap : L - 1;
    append = p.k_new != nullptr && start <= slot_new && slot_new < end;
  }
  if constexpr (FUSED || BLOCK) {
    if (append) {
      // the new key, normalised and rotated by the same row code as the
      // append kernel, and the new value, into slot len-1 (or its ring
      // slot); 16 lanes per row, only the first row is real.  The V^T area
      // is free until the key loop.
      float* xs = reinterpret_cast<float*>(smem);
      float* cs = xs + 16 * kD;
      float* sn = cs + 16 * kMaxRopeHalf;
      const int lrow = tid >> 4, c16 = tid & 15;
      const long long row = (long long)b * p.Hkv + g;
      float x[8];
      u32x4 vv = {0, 0, 0, 0};
      if (lrow == 0) {
        unpack_bf16x8(ld16(p.k_new + row * kD + 8 * c16), x);
        vv = ld16(p.v_new + row * kD + 8 * c16);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
      }
      norm_rope_row(x, c16, p.k_norm_w, p.eps, p.rope_half, p.tab, pos, xs + lrow * kD, true,
                    cs + lrow * kMaxRopeHalf, sn + lrow * kMaxRopeHalf, cs + lrow * kMaxRopeHalf,
                    sn + lrow * kMaxRopeHalf);
      if (lrow == 0) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        const int slot = p.ring ? (L - 1) % p.cap : L - 1;
        long long dst;
        if (PAGED) {
          const int pg = p.map.page(b, slot);
          dst = ((((long long)pg * p.Hkv + g) << psh) + (slot & ((1 << psh) - 1))) * kD;
        } else {
          dst = (row * p.cap + slot) * kD;
        }
        if constexpr (FP8) {
          float vf[8];
          unpack_bf16x8(vv, vf);
          uint8_t* kc = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.k_cache));
          uint8_t* vc = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.v_cache));
          st8(kc + dst + 8 * c16, pack_e4m3x8(x, p.k_scale));
          st8(vc + dst + 8 * c16, pack_e4m3x8(vf, p.v_scale));
        } else {
          st16(const_cast<uint16_t*>(p.k_cache) + dst + 8 * c16, o);
          st16(const_cast<uint16_t*>(p.v_cache) + dst + 8 * c16, vv);
        }
      }
      // The key loop below reads the slot back.  All waves of the workgroup
      // share the CU's vector cache, so the barrier's workgroup-scope
      // release / acquire (stores complete first) is enough; the slot's
      // cache lines belong to this (b, kv head) alone.
      __syncthreads();
    }
  }

  // ---- query prologue for the group's heads (RMSNorm, partial RoPE)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wv + kWaves * j;
    if (c >= grp) break;
    const float x0 = xq[j][0], x1 = xq[j][1];
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
    qn[c * kD + lane] = x0 * r * p.q_norm_w[lane];
    qn[c * kD + 64 + lane] = x1 * r * p.q_norm_w[64 + lane];
  }
  __syncthreads();
  for (int idx = tid; idx < 16 * kD; idx += kThreads) {
    const int c = idx / kD, d = idx % kD;
    float v = 0.f;
    if (c < grp) {
      v = qn[c * kD + d];
      if (d < 2 * p.rope_half) {
        const int t = d < p.rope_half ? d : d - p.rope_half;
        float cs, sn;
        rope_cos_sin(p.tab, t, pos, cs, sn);
        v = d < p.rope_half ? v * cs - qn[c * kD + d + p.rope_half] * sn
                            : v * cs + qn[c * kD + d - p.rope_half] * sn;
      }
    }
    if constexpr (FP8) reinterpret_cast<float*>(smem)[c * kD + d] = v;  // V^T area: free here
    else qs[c * kQsStride + d] = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  __syncthreads();
  bf16x8 qf[4];
  i32x8 qb;          // FP8: this lane's B operand, codes of dims 32kg..32kg+31 of head col
  float qinv = 1.f;  // FP8: 1 / (that head's query scale)
  if constexpr (FP8) {
    // each head's row of Q' to E4M3 with the power-of-two scale 2^(8-e),
    // amax = m 2^e (m in [0.5, 1), e >= -100): 16 threads per row, 8 dims each
    const float* qr = reinterpret_cast<const float*>(smem);
    const int c = tid >> 4, part = tid & 15;
    float x8[8];
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x8[i] = qr[c * kD + 8 * part + i];
      am = fmaxf(am, fabsf(x8[i]));
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 16));
    int e;
    frexpf(am, &e);
    e = max(e, -100);
    uint8_t* q8 = reinterpret_cast<uint8_t*>(qs);
    st8(q8 + c * kD + 8 * part, pack_e4m3x8(x8, ldexpf(1.0f, 8 - e)));
    if (part == 0) qn[c] = ldexpf(1.0f, e - 8);  // qn is dead after the rotation
    __syncthreads();
    const u32x4 lo = ld16(q8 + col * kD + 32 * kg), hi = ld16(q8 + col * kD + 32 * kg + 16);
    qb = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    qinv = qn[col];
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qs + col * kQsStride + 32 * kk + 8 * kg);
  }
  // score scale in exp2 units of this lane's head
  const float sl2 = FP8 ? p.scale_log2 * qinv : p.scale_log2;

  // ---- stream the split's keys.  Cache row of key `key` relative to the
  // cache base: a contiguous slab per (b, kv head), or the key's page slot
  // (a wave's 32-key slice spans at most two pages, looked up once per
  // slice: pa for the slice's first key, pb for its last)
  const long long slab = ((long long)b * p.Hkv + g) * p.cap * kD;
  auto row_off = [&](int key, int pa, int pb, int base) -> long long {
    if (!PAGED) return slab + (long long)key * kD;
    const int pg = (key >> psh) == (base >> psh) ? pa : pb;
    return (((long long)pg * p.Hkv + g) << psh) * kD + (long long)(key & ((1 << psh) - 1)) * kD;
  };
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  uint16_t* vt = vt_all + wv * kD * kVtwStride;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const int nit = end > start ? (end - start + kKeysPerIter - 1) / kKeysPerIter : 0;
  const int mr = lane & 15;
  const int krel = 8 * (mr >> 2) + (mr & 3);  // + 4*blk: key of MFMA row mr
  const float rescale_raw = kRescaleThreshold / sl2;

  // The raw cache bytes of the next kDepth slices are in flight while a
  // slice is processed, so that a wave keeps loads moving during its MFMAs
  // and softmax.  bf16: one slice ahead, the operands themselves (64
  // registers); FP8: two slices ahead, the codes (32 registers per slice),
  // widened after arrival, since a slice of codes is half the bytes.
  constexpr int kDepth = FP8 ? 2 : 1;
  constexpr int kRawK = FP8 ? 2 : 4;  // 16-byte loads per key row and lane
  u32x4 rk[kDepth][2][kRawK];
  u32x4 rv16[kDepth][FP8 ? 1 : 8];
  uint2 rv8[kDepth][FP8 ? 8 : 1];
  // Keys past the range load row min(key, end - 1) instead: a visible,
  // written row, so its values are finite; its score is replaced by -inf
  // below, so it adds exact zeros (the loads need no branch).
  auto load_slice = [&](int it2, int d) {
    const int b2 = start + it2 * kKeysPerIter + wvu * kKeysPerWave;  // wave-uniform
    int qa = 0, qb = 0;
    if (PAGED && b2 < end) {
      qa = p.map.page(b, b2);
      qb = p.map.page(b, min(b2 + kKeysPerWave - 1, end - 1));
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const long long ro = row_off(min(b2 + krel + 4 * blk, end - 1), qa, qb, b2);
      if constexpr (FP8) {
        // bytes 32kg..32kg+31 of the key row: dims 32kg + 8kk + 0..7 of kf[kk]
        const uint8_t* src = reinterpret_cast<const uint8_t*>(p.k_cache) + ro + 32 * kg;
        rk[d][blk][0] = ld16(src);
        rk[d][blk][1] = ld16(src + 16);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) rk[d][blk][kk] = ld16(p.k_cache + ro + 32 * kk + 8 * kg);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const long long ro = row_off(min(b2 + 8 * kg + j, end - 1), qa, qb, b2);
      if constexpr (FP8)
        rv8[d][j] = ld8(reinterpret_cast<const uint8_t*>(p.v_cache) + ro + 8 * col);
      else
        rv16[d][j] = ld16(p.v_cache + ro + 8 * col);
    }
  };
  // Every prefetch is issued, also past the last slice (it then re-reads
  // slice nit - 1, an L2 hit): a conditional one would make the compiler
  // copy the buffers at the loop head, waiting for all loads in flight.
  if (nit > 0) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_slice(min(d, nit - 1), d);
  }

  // With kDepth 2 an odd slice count ends with slice nit, past the range:
  // all its keys are masked, so it adds exact zeros and leaves the max.
  for (int it0 = 0; it0 < nit; it0 += kDepth)
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int it = it0 + d;
    const int base = start + it * kKeysPerIter + wvu * kKeysPerWave;  // wave-uniform
    bf16x8 kf[2][4];
    u32x4 vr[8];
    f32x4 s[2];
    if constexpr (FP8) {
      // S^T = K' Q'^T on the FP8 matrix cores: the key codes as they came
      // (row krel, bytes 32kg..32kg+31) against the query codes, one
      // 16 x 16 x 128 product per 16 keys; block scales 1 (E8M0 127)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const u32x4& lo = rk[d][blk][0];
        const u32x4& hi = rk[d][blk][1];
        const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, f32x4{}, 0, 0, 0, 127,
                                                                  0, 127);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j] = widen_e4m3x8(rv8[d][j]);
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[blk][kk] = __builtin_bit_cast(bf16x8, rk[d][blk][kk]);
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j] = rv16[d][j];
    }
    // the buffer's old contents are consumed before its refill is issued,
    // so the refill lands in the same registers (no copies at the loop end)
    __builtin_amdgcn_sched_barrier(0);
    load_slice(min(it + kDepth, nit - 1), d);

    if constexpr (!FP8) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        s[blk] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[blk][kk], qf[kk], s[blk], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = base + 8 * kg + 4 * blk + e;
        const float v = key < end ? s[blk][e] : -INFINITY;
        s[blk][e] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + rescale_raw)) {
      const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2((m_run - m_new) * sl2);
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg_mc = m_run == -INFINITY ? 0.0f : -m_run * sl2;
    float pv[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[4 * blk + e] = fast_exp2(__builtin_fmaf(s[blk][e], sl2, neg_mc));
        l_run += pv[4 * blk + e];
      }
    }
    const bf16x8 pf = pack_bf16x8(pv);

    // V slice (keys 8kg..8kg+7, dims 8col..8col+7 per lane) -> V^T tile
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int wd = i >> 1;
      u32x4 t;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t a = vr[2 * q2][wd], c = vr[2 * q2 + 1][wd];
        t[q2] = (i & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      st16(vt + (8 * col + i) * kVtwStride + 8 * kg, t);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (16 * db + mr) * kVtwStride + 8 * kg);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, o[db], 0, 0, 0);
    }
  }

  // ---- combine the four waves, write this split's partial
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // V^T tiles are dead; reuse them for red_o
  if (kg == 0) {
    red_m[wv][col] = m_run == -INFINITY ? -INFINITY : m_run * sl2;
    red_l[wv][col] = l_run;
  }
  if (col < grp) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red_o[(wv * kMaxGroup + col) * kD + 16 * db + 4 * kg + e] = o[db][e];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaxGroup * kD / kThreads; ++j) {
    const int idx = tid + j * kThreads;
    if (idx >= grp * kD) break;
    const int c = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, red_m[w2][c]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const float mw = red_m[w2][c];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      acc += f * red_o[(w2 * kMaxGroup + c) * kD + d];
      lsum += f * red_l[w2][c];
    }
    if constexpr (FP8) acc *= p.v_inv;
    if constexpr (FUSED) {
      // what the merge computes for one split (its weight is exactly 1)
      const long long oi = ((long long)b * p.Hq + g * grp + c) * kD + d;
      float o = acc * (1.0f / lsum);
      if (p.gate) o *= sigmoidf_(gpre[j]);
      p.out[oi] = __builtin_bit_cast(uint16_t, (__bf16)o);
    } else {
      const long long pi = ((long long)b * p.Hq + g * grp + c) * p.nsplit + split;
      if constexpr (BLOCK) {  // device-coherent stores (see the merge below)
        store_coherent(p.part_o + pi * kD + d, acc);
        if (d == 0) {
          store_coherent(p.part_ml + 2 * pi, M);
          store_coherent(p.part_ml + 2 * pi + 1, lsum);
        }
      } else {
        p.part_o[pi * kD + d] = acc;
        if (d == 0) {
          p.part_ml[2 * pi] = M;
          p.part_ml[2 * pi + 1] = lsum;
        }
      }
    }
  }
  if constexpr (BLOCK && !FUSED) {
    // Publish the partial and take a ticket; the last split of this (b, kv
    // head) merges.  The splits run on every XCD, each with its own L2, so
    // the partials cross workgroups only through device-coherent accesses:
    // they are stored write-through (agent-scope atomic stores), every
    // thread waits for its stores to complete before the barrier, and only
    // then does thread 0 take the ticket; the merging workgroup reads them
    // with device-coherent loads.  No plain data crosses workgroups, so no
    // L2 writeback or invalidate (a device-scope fence) is needed: those
    // cost about a microsecond each, and a step has a thousand workgroups.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      unsigned* t = p.tickets + (long long)b * p.Hkv + g;
      const unsigned done = atomicAdd(t, 1u) + 1u;
      const int last = done == (unsigned)p.nsplit;
      if (last) atomicExch(t, 0u);
      lds.last = last;
    }
    __syncthreads();
    if (lds.last) {
      // the arithmetic of decode_merge_kernel, element by element
      for (int idx = tid; idx < grp * kD; idx += kThreads) {
        const int c = idx / kD, d = idx % kD;
        const long long bh = (long long)b * p.Hq + g * grp + c;
        const float* ml = p.part_ml + bh * p.nsplit * 2;
        const float* po = p.part_o + bh * p.nsplit * kD;
        float M = -INFINITY;
        for (int s2 = 0; s2 < p.nsplit; ++s2) M = fmaxf(M, load_coherent(ml + 2 * s2));
        float a = 0.f, lsum = 0.f;
        for (int s2 = 0; s2 < p.nsplit; ++s2) {
          const float ms = load_coherent(ml + 2 * s2);
          const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
          lsum += f * load_coherent(ml + 2 * s2 + 1);
          a += f * load_coherent(po + (long long)s2 * kD + d);
        }
        const float inv = 1.0f / lsum;
        float o = a * inv;
        if (p.gate) o *= sigmoidf_(__uint_as_float((uint32_t)p.gate[bh * kD + d] << 16));
        p.out[bh * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
      }
    }
  }
}

template <bool PAGED, bool FUSED, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeParams p) {
  __shared__ DecodeLds lds;
  decode_split_body<PAGED, FUSED, FP8, false>(p, blockIdx.x, lds);
}

// One decode step of a block of layers in a single launch: workgroups
// [wg0[l], wg0[l + 1]) are layer l's (b, kv head, split) workgroups, bf16
// contiguous caches.  Each layer's parameters are read in place from the
// kernel arguments.
__global__ __launch_bounds__(kThreads, 2) void decode_block_kernel(DecodeBlockParams bp) {
  __shared__ DecodeLds lds;
  const int bid = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxBlockLayers; ++i)
    if (i < bp.n_layers && bid >= bp.wg0[i]) l = i;
  const DecodeParams& p = bp.layer[l];
  if (p.nsplit == 1) decode_split_body<false, true, false, true>(p, bid - bp.wg0[l], lds);
  else decode_split_body<false, false, false, true>(p, bid - bp.wg0[l], lds);
}

__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;  // b * Hq + h
  const int lane = threadIdx.x;
  const float* ml = p.part_ml + (long long)bh * p.nsplit * 2;
  const float* po = p.part_o + (long long)bh * p.nsplit * kD;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float a0 = 0.f, a1 = 0.f, lsum = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float ms = ml[2 * s];
    const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    lsum += f * ml[2 * s + 1];
    a0 += f * po[(long long)s * kD + lane];
    a1 += f * po[(long long)s * kD + 64 + lane];
  }
  const float inv = 1.0f / lsum;
  float o0 = a0 * inv, o1 = a1 * inv;
  if (p.gate) {
    const uint16_t* gs = p.gate + (long long)bh * kD;
    o0 *= sigmoidf_(__uint_as_float((uint32_t)gs[lane] << 16));
    o1 *= sigmoidf_(__uint_as_float((uint32_t)gs[64 + lane] << 16));
  }
  uint16_t* dst = p.out + (long long)bh * kD;
  dst[lane] = __builtin_bit_cast(uint16_t, (__bf16)o0);
  dst[64 + lane] = __builtin_bit_cast(uint16_t, (__bf16)o1);
}

template <bool FUSED>
void launch_split(const DecodeParams& p, bool paged, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.fp8) {
    if (paged) hipLaunchKernelGGL((decode_split_kernel<true, FUSED, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_split_kernel<false, FUSED, true>), grid, block, 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((decode_split_kernel<true, FUSED, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_split_kernel<false, FUSED, false>), grid, block, 0, stream, p);
  }
}

}  // namespace

hipError_t launch_decode_block(const DecodeBlockParams& bp, int total_wgs, hipStream_t stream) {
  if (total_wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_block_kernel, dim3((unsigned)total_wgs), dim3(kThreads), 0, stream, bp);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  const long long blocks = (long long)p.B * p.Hkv * p.nsplit;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kThreads);
  const bool paged = p.map.block_table != nullptr;
  if (p.nsplit == 1) {
    launch_split<true>(p, paged, grid, block, stream);
    return hipGetLastError();
  }
  launch_split<false>(p, paged, grid, block, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(p.B * p.Hq), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace zg
