// Host-side launchers of the libzgattn kernels (internal; the public C ABI
// is include/zg_attn.h).  Every launcher enqueues on `stream` and returns the
// launch status without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zg_common.h"

namespace zg {

struct FlashParams {
  const uint16_t* q;     // bf16 [B,S,Hq,D] raw queries
  const uint16_t* kp;    // bf16 [B,S,Hkv,D] normalised + rotated keys
  // E4M3 variant (kp8 != null, global layers): the keys as E4M3 codes of
  // K' * k_scale [B,S,Hkv,D], one byte each; kp is then unused
  const uint8_t* kp8;
  float k_scale;
  const uint16_t* v;     // bf16 [B,S,Hkv,D]
  const uint16_t* gate;  // bf16 [B,S,Hq,D] or null
  const float* q_norm_w; // fp32 [D]
  const float* k_norm_w; // fp32 [D] (the causal kernel bounds its scores with it)
  uint16_t* out;         // bf16 [B,S,Hq,D]
  float* lse;            // fp32 [B,Hq,S], or [Hq,total] when packed; or null
  int B, S, Hq, Hkv, window, rope_half;
  float scale_log2;      // softmax scale * log2(e)
  float eps;
  long long pos_offset;
  RopeTable tab;
  // Packed variable-length batch: rows [cu_seqlens[b], cu_seqlens[b+1]) of
  // the token-major tensors form sequence b; S is then the longest length
  // (it sizes the grid) and total the number of rows.  Null: B fixed-length
  // sequences of S tokens.
  const int* cu_seqlens;
  long long total;
  // Global (causal) layers: 16 int32 work-queue counters in device memory,
  // zero when the kernel starts (the key prologue clears them) and left
  // nonzero by it.  Launches that overlap on one set of counters race.
  int* queue;
};

// Rows are (token, head) of a token-major [tokens, H, D] tensor.  Token t
// sits at position pos_offset + (t mod S), or, with cu_seqlens (int32
// [nseq + 1] on the device), pos_offset + t - cu_seqlens[b] for the sequence
// b that holds it.  kout receives K' * out_scale in bf16 (rounded once).
// zero16, if not null, points at 16 int32 that the launch sets to zero (the
// causal kernel's work-queue counters, FlashParams::queue).
hipError_t launch_k_prologue(const uint16_t* k, const float* w, uint16_t* kout, long long rows,
                             int S, int Hkv, long long pos_offset, int rope_half, float eps,
                             const RopeTable& tab, hipStream_t stream,
                             const int* cu_seqlens = nullptr, int nseq = 0,
                             float out_scale = 1.0f, int* zero16 = nullptr);

// The same with K' written as the E4M3 codes of K' * k_scale (one byte per
// element: product in fp32, clamped to +-448, rounded to nearest even).
hipError_t launch_k_prologue_fp8(const uint16_t* k, const float* w, uint8_t* kout, float k_scale,
                                 long long rows, int S, int Hkv, long long pos_offset,
                                 int rope_half, float eps, const RopeTable& tab,
                                 hipStream_t stream, const int* cu_seqlens = nullptr,
                                 int nseq = 0, int* zero16 = nullptr);

hipError_t launch_flash_fwd(const FlashParams& p, hipStream_t stream);
// The global (window 0) layer's kernel; launch_flash_fwd routes to it.
hipError_t launch_flash_causal(const FlashParams& p, hipStream_t stream);

// Where a sequence's cache rows live.  Contiguous: one slab [cap, D] per
// (b, kv head).  Paged (block_table != null): token t of sequence b is slot
// t % page_size of page block_table[b * max_pages + t / page_size], and a
// page holds [Hkv, page_size, D]; page_size is a power of two >= 32.
// Paged KV cache: page table row b lists the pages of sequence b; key slot t
// sits in page table[b][t >> page_shift], row t & (page_size-1) of that
// page's [Hkv, page_size, D] block.  Page ids are clamped into [0, num_pages)
// so a bad table entry cannot address memory outside the pool.
struct CacheMap {
  const int* block_table;  // int32 [B, max_pages], or null: contiguous slabs
  int max_pages;
  int page_shift;  // log2(page_size)
  int num_pages;

  __device__ __forceinline__ int page(long long b, int slot) const {
    const int pg = block_table[b * max_pages + (slot >> page_shift)];
    return (int)min((unsigned)pg, (unsigned)(num_pages - 1));
  }
};

// fp8 != 0: the caches hold E4M3 codes (one byte per element) of
// K' * k_scale and V * v_scale.
hipError_t launch_decode_append(const uint16_t* k_new, const uint16_t* v_new, void* k_cache,
                                void* v_cache, const int* seq_lens, const float* w, int B,
                                int Hkv, int cap, int ring, const CacheMap& map,
                                long long pos_offset, int rope_half, float eps,
                                const RopeTable& tab, int fp8, float k_scale, float v_scale,
                                hipStream_t stream);

// Copy K' and V of a prefill (bf16 [B,S,Hkv,D]) into a paged cache: token s
// of sequence b goes to its page slot (CacheMap).
hipError_t launch_kv_write_pages(const uint16_t* kp, const uint16_t* v, uint16_t* k_pages,
                                 uint16_t* v_pages, int B, int S, int Hkv, const CacheMap& map,
                                 hipStream_t stream);

struct DecodeParams {
  const uint16_t* q;        // bf16 [B,Hq,D] raw
  const uint16_t* k_cache;  // bf16 [B,Hkv,cap,D], or pages [num_pages,Hkv,page,D]
  const uint16_t* v_cache;  // bf16, same layout as k_cache
  const int* seq_lens;      // int32 [B]
  const float* q_norm_w;    // fp32 [D]
  const uint16_t* gate;     // bf16 [B,Hq,D] or null
  uint16_t* out;            // bf16 [B,Hq,D]
  float* part_o;            // fp32 [B,Hq,nsplit,D]
  float* part_ml;           // fp32 [B,Hq,nsplit,2]
  int B, Hq, Hkv, cap, ring, window, nsplit, rope_half;
  float scale_log2, eps;
  long long pos_offset;
  CacheMap map;             // block_table == null: contiguous slabs
  // With a single split the split kernel is the whole step: it appends the
  // new token (when k_new is given), attends and writes `out` itself.
  const uint16_t* k_new;    // bf16 [B,Hkv,D] raw, or null
  const uint16_t* v_new;    // bf16 [B,Hkv,D]
  const float* k_norm_w;    // fp32 [D]
  RopeTable tab;
  // E4M3 cache (the FP8 instance): k_cache / v_cache hold codes, one byte
  // per element in the same layouts, of K' * k_scale and V * v_scale.  The
  // launch folds 1 / k_scale into scale_log2; v_inv = 1 / v_scale.
  float k_scale, v_scale, v_inv;
  int fp8;
  // block launch (launch_decode_block), several splits: one ticket counter
  // per (b, kv head)
  unsigned* tickets;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// A decode step of several layers in one launch (bf16 contiguous caches):
// each layer's full parameters (its split count, workspace segments and, for
// several splits, its tickets: one counter per (b, kv head), zero between
// steps), and the first workgroup of each layer (ascending).
constexpr int kMaxBlockLayers = 6;
struct DecodeBlockParams {
  DecodeParams layer[kMaxBlockLayers];
  int wg0[kMaxBlockLayers];
  int n_layers;
};
hipError_t launch_decode_block(const DecodeBlockParams& bp, int total_wgs, hipStream_t stream);


// Projections: C = A B^T with A [M, K] and B [N, K] bf16 row major (row
// strides lda, ldb elements); output columns [seg[i].n0, seg[i+1].n0) go to
// seg[i].ptr with row stride seg[i].ld.  Segment starts are sorted and
// multiples of 256; N is a multiple of 256 and K of 32.
constexpr int kGemmMaxSegs = 4;
struct GemmSeg {
  uint16_t* ptr;
  int n0;
  int ld;
};
struct GemmParams {
  const uint16_t* a;
  const uint16_t* b;
  int M, N, K;
  int lda, ldb;
  GemmSeg seg[kGemmMaxSegs];
  int nseg;
  int fp8;           // operands are FP8 E4M3 bytes (K a multiple of 128)
  float out_scale;   // fp8: results are multiplied by this before rounding
  int tiles_m, tiles_n;  // set by the launcher
};

hipError_t launch_gemm_bf16_tn(GemmParams p, hipStream_t stream);
// n bf16 values -> FP8 E4M3 bytes, q = RNE(clamp(x * scale, +-448)); n % 8 == 0
hipError_t launch_quantize_fp8(const uint16_t* x, uint8_t* q, long long n, float scale,
                               hipStream_t stream);

// Training backward.  The prep launch recomputes K' (KPrimeJob).  The score
// operand Q' * c (c = softmax scale * log2 e, as in the forward) is formed by
// the dq' kernel where it fuses the query prologue (bwd_dq_fuses_q), else by
// launch_k_prologue with out_scale c; either way it lands in qp, where the
// dk'/dv kernel reads it.  dO = dY * sigmoid(G) (dY itself on an ungated layer).
// The dq' and dk'/dv kernels finish with the RoPE / RMSNorm backward of their
// rows: they write dq and dk, and one partial sum of the norm-weight gradient
// per workgroup (part_q, part_k), which launch_reduce_parts adds up.
struct BwdParams {
  const uint16_t* qp;   // bf16 [B,S,Hq,D]   Q' * c, the score operand
  const uint16_t* kp;   // bf16 [B,S,Hkv,D]  K'
  const uint16_t* v;    // bf16 [B,S,Hkv,D]
  const uint16_t* dO;   // bf16 [B,S,Hq,D]
  const float* nlse2;   // fp32 [B,Hq,Spad]  -LSE * log2(e); -inf for rows >= S
  const float* dvec;    // fp32 [B,Hq,Spad]  rowsum(dY * Y); 0 for rows >= S
  uint16_t* dq;         // bf16 [B,S,Hq,D]
  uint16_t* dk;         // bf16 [B,S,Hkv,D]
  uint16_t* dv;         // bf16 [B,S,Hkv,D]
  float* part_q;        // fp32 [bwd_dq_blocks][D]   partial d(q_norm_w)
  float* part_k;        // fp32 [bwd_dkv_blocks][D]  partial d(k_norm_w)
  int B, S, Spad, Hq, Hkv, window;
  float scale_log2;     // softmax scale * log2(e)
  float scale;          // softmax scale
  const uint16_t* q;    // bf16 [B,S,Hq,D]   raw q (the dq' kernel's Q' and RMSNorm backward)
  const uint16_t* k;    // bf16 [B,S,Hkv,D]  raw k (the dk' RMSNorm backward)
  const float* q_norm_w;
  const float* k_norm_w;
  float eps;
  int rope_half;
  long long pos_offset;
  RopeTable tab;
};

// The dq' kernel forms Q' itself, with the forward's fused query prologue,
// when the rotation runs in registers there (rope_dim 42 or 0).
inline bool bwd_dq_fuses_q(int rope_half) { return rope_half == 21 || rope_half == 0; }

// Row padding of the LSE / D vectors (a multiple of every query block).
constexpr int kBwdRowPad = 128;

// Grid of the dq' kernel: a workgroup is (batch, kv head, group of hpw query
// heads, ppw positions), hpw * ppw = 128 rows.
struct DqGeo {
  int hpw;  // query heads per workgroup
  int ppw;  // query positions per workgroup
  int n_pos_blocks, hgroups, n_bhg;
};
inline DqGeo bwd_dq_geo(int B, int S, int Hq, int Hkv) {
  const int grp = Hq / Hkv;
  DqGeo geo;
  geo.hpw = grp < 4 ? grp : 4;
  geo.hgroups = grp / geo.hpw;
  geo.ppw = 128 / geo.hpw;
  geo.n_pos_blocks = (S + geo.ppw - 1) / geo.ppw;
  geo.n_bhg = B * Hkv * geo.hgroups;
  return geo;
}
inline long long bwd_dq_blocks(int B, int S, int Hq, int Hkv) {
  const DqGeo g = bwd_dq_geo(B, S, Hq, Hkv);
  return (long long)g.n_pos_blocks * g.n_bhg;
}
// The dk'/dv kernel: a workgroup is (batch, kv head, 128 keys).
inline long long bwd_dkv_blocks(int B, int S, int Hkv) {
  return (long long)((S + 127) / 128) * B * Hkv;
}
// First stage of the weight-gradient sum: this many fixed chunks of partials
// per gradient, summed in order, then the chunk sums in order.
constexpr int kBwdRedChunks = 256;

// K' recomputed inside the prep launch: rows = B * S * Hkv key rows of k
// (token-major, heads innermost) through RMSNorm (weight w) + partial RoPE
// into kout, with the key prologue's row code.  blocks is set by the launch.
struct KPrimeJob {
  const uint16_t* k;
  const float* w;
  uint16_t* kout;
  long long rows;
  int S, Hkv;
  long long pos_offset;
  int rope_half;
  float eps;
  RopeTable tab;
  long long blocks;
};
hipError_t launch_bwd_prep(const uint16_t* dy, const uint16_t* y, const uint16_t* gate,
                           const float* lse, uint16_t* dO, uint16_t* dgate, float* nlse2,
                           float* dvec, int B, int S, int Spad, int Hq, KPrimeJob kp,
                           hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdParams& p, hipStream_t stream);
// d(q_norm_w) and d(k_norm_w) from the kernels' partials, in a fixed order;
// red: fp32 [2][kBwdRedChunks][D] scratch.
hipError_t launch_reduce_parts(const BwdParams& p, float* red, float* dwq, float* dwk,
                               hipStream_t stream);

}  // namespace zg
