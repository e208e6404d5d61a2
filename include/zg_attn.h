/*
 * zg_attn — gated sliding-window + global causal attention of the ZGCM-1
 * decoder, for AMD Instinct MI355X (gfx950).  C ABI of libzgattn.so.
 *
 * What is computed (pages cited by title and section):
 *  - "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型" (paper.rainbus.top),
 *    section 前置知识 › 滑动窗口注意力(SWA)与混合注意力: each token attends
 *    only to its 128 neighbouring tokens (the sliding-window layers); global
 *    layers at 6/12/18/24/30 of 32 attend over the whole causal prefix.
 *    Section 核心方法: GQA with 32 query / 8 KV heads, partial RoPE ratio 0.33.
 *  - "7B 打 235B？中关村学院把'小模型怎么活'这道题答成了一份全开源配方"
 *    (shibing624.github.io), section 🏗️ 架构: QK normalised with RMSNorm;
 *    the local (sliding-window) attention output is multiplied by a sigmoid
 *    gate.
 *
 * Per query row i of query head h (kv head g = h / (n_q_heads/n_kv_heads)):
 *   q' = RoPE(RMSNorm(q_i) * q_norm_w),  k'_j = RoPE(RMSNorm(k_j) * k_norm_w)
 *   RMSNorm(x) = x / sqrt(mean(x^2) + rms_eps) over the head_dim values;
 *   RoPE rotates dims (t, t + rope_dim/2), t < rope_dim/2, by the angle
 *   p * rope_theta^(-2t/rope_dim) at position p = pos_offset + i; other dims
 *   pass through.
 *   key j visible iff j <= i and (window == 0 or i - j < window);
 *   out_i = softmax_j(scale * q'.k'_j) V_j, then out_i *= sigmoid(gate_i)
 *   elementwise when a gate is given;  lse_i = log sum_j exp(scale q'.k'_j).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, 16-byte aligned, contiguous in the
 *    documented layout; bf16 means IEEE bfloat16 bits.  The caller owns all
 *    buffers; the library allocates nothing and keeps no pointer after return.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising.  No global mutable state:
 *    calls from several host threads are safe.
 *  - Arguments are validated before anything is launched; on error nothing
 *    is launched and a negative status is returned (no exceptions cross the
 *    ABI).
 */
#ifndef ZG_ATTN_H
#define ZG_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZG_OK               0
#define ZG_ERR_INVALID     -1  /* null pointer, bad shape, misaligned pointer  */
#define ZG_ERR_UNSUPPORTED -2  /* valid but not implemented (head_dim != 128,
                                  rope_dim > head_dim/2, odd rope_dim, ...)    */
#define ZG_ERR_WORKSPACE   -3  /* workspace missing or smaller than required   */
#define ZG_ERR_HIP         -4  /* a HIP launch or runtime call failed          */
#define ZG_ERR_TOO_LARGE   -5  /* more scratch than zg_attn_decode_noalloc holds */

typedef struct zg_attn_params {
  int   batch;          /* B  (>= 0)                                            */
  int   seqlen;         /* S: tokens per sequence (fwd); ignored by decode     */
  int   n_q_heads;      /* Hq (32 in ZGCM-1)                                    */
  int   n_kv_heads;     /* Hkv (8); Hq % Hkv == 0 and Hq/Hkv in {1,2,4,8}      */
  int   head_dim;       /* D; must be 128                                      */
  int   window;         /* 0 = global causal; W > 0: key j visible to query i
                           iff 0 <= i - j < W (128 for the SWA layers)         */
  int   rope_dim;       /* rotary dims R: even, 0 <= R <= head_dim/2 (42)      */
  float rope_theta;     /* RoPE base (10000; 1e7 for the 256K stage)           */
  float rms_eps;        /* RMSNorm epsilon (1e-6)                              */
  float softmax_scale;  /* 0 -> 1/sqrt(head_dim)                               */
  long long pos_offset; /* position of token 0 (fwd) / added to decode pos.    */
} zg_attn_params;

/* Bytes of device workspace zg_attn_fwd needs (16-byte aligned): the
 * normalised and rotated keys K', bf16 [B,S,Hkv,D], and for a global layer
 * (window 0) after them, on the next 256-byte boundary, 256 bytes of work-
 * queue counters that the call clears before its attention kernel uses them;
 * 0 for an invalid p or an empty batch.  When k_out is passed, K' goes there:
 * a windowed layer then needs no workspace (NULL is fine), a global layer 256
 * bytes for the counters.  Calls that run at the same time need workspaces
 * of their own. */
size_t zg_attn_fwd_workspace_size(const zg_attn_params* p);

/* Prefill / training forward of one attention layer.
 *   q     bf16 [B,S,Hq,D]   raw queries (before norm / RoPE)
 *   k     bf16 [B,S,Hkv,D]  raw keys
 *   v     bf16 [B,S,Hkv,D]
 *   gate  bf16 [B,S,Hq,D]   gate logits (out *= sigmoid(gate)), or NULL
 *   q_norm_w, k_norm_w  fp32 [D] RMSNorm weights
 *   out   bf16 [B,S,Hq,D]   written in full
 *   lse   fp32 [B,Hq,S]     natural-log LSE of the scaled scores, or NULL
 *   k_out bf16 [B,S,Hkv,D]  receives K' (for filling a KV cache), or NULL
 * S == 0 or B == 0 is valid and launches nothing. */
int zg_attn_fwd(const zg_attn_params* p,
                const void* q, const void* k, const void* v, const void* gate,
                const float* q_norm_w, const float* k_norm_w,
                void* out, float* lse, void* k_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Packed variable-length prefill: the same attention as zg_attn_fwd over a
 * batch of sequences of different lengths stored back to back, as a server
 * batches prompts (the ZGCM-1 page's structured-data table, row
 * "256K 上下文推理 KV 缓存", and its section 核心方法 describe the serving
 * setting; the pages fix no batching format, so this is the common
 * cumulative-offsets one).
 *   p->batch      number of sequences B
 *   p->seqlen     an upper bound on every length (sizes the grid); rows of a
 *                 longer sequence past p->seqlen are not computed
 *   cu_seqlens    device int32 [B+1]: sequence b is rows
 *                 [cu_seqlens[b], cu_seqlens[b+1]) (0 = cu_seqlens[0] <= ...
 *                 <= cu_seqlens[B] = total_tokens); empty sequences allowed.
 *                 Read on the device and clamped into [0, total_tokens].
 *   q, gate, out  bf16 [total_tokens,Hq,D];  k, v, k_out bf16 [total_tokens,Hkv,D]
 *   lse           fp32 [Hq,total_tokens] or NULL
 * Token s of every sequence sits at position pos_offset + s.  Each sequence's
 * rows are bit-identical to zg_attn_fwd on that sequence alone. */
/* Workspace as for zg_attn_fwd, with total_tokens rows of K'. */
size_t zg_attn_fwd_varlen_workspace_size(const zg_attn_params* p, long long total_tokens);
int zg_attn_fwd_varlen(const zg_attn_params* p, const int* cu_seqlens, long long total_tokens,
                       const void* q, const void* k, const void* v, const void* gate,
                       const float* q_norm_w, const float* k_norm_w,
                       void* out, float* lse, void* k_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Number of KV splits zg_attn_decode uses when num_splits == 0. */
int zg_attn_decode_num_splits(const zg_attn_params* p, int cache_cap);

/* Bytes of device workspace zg_attn_decode needs for `num_splits` splits
 * (0 = the automatic choice): fp32 partial (max, sum, acc[D]) per
 * (b, q head, split).  0 for an invalid p. */
size_t zg_attn_decode_workspace_size(const zg_attn_params* p, int cache_cap, int num_splits);

/* One decode step: one new token per sequence against a KV cache.
 *   q         bf16 [B,Hq,D]   raw new-token queries
 *   k_new     bf16 [B,Hkv,D]  raw new key, or NULL if the cache already holds
 *   v_new     bf16 [B,Hkv,D]  the new token's K' and V (then both NULL)
 *   k_cache   bf16 [B,Hkv,cache_cap,D]  K' (post norm/RoPE), updated in place
 *   v_cache   bf16 [B,Hkv,cache_cap,D]  V, updated in place
 *   seq_lens  device int32 [B]: tokens of each sequence INCLUDING the new
 *             one (>= 1); the query sits at position pos_offset+len-1
 *   ring      0: slot = position (len <= cache_cap required);
 *             1: slot = position % cache_cap (sliding-window ring; requires
 *                window == cache_cap)
 *   gate      bf16 [B,Hq,D] or NULL;  out bf16 [B,Hq,D]
 *   num_splits  KV splits per (b, kv head); 0 = automatic
 * Visible keys: positions max(0,len-W)..len-1 (W = window, or all for 0).
 * The new token's K' and V are written to their slot before attending.
 * seq_lens values are read on the device; values outside [1, cache_cap] for
 * ring == 0 are clamped to that range. */
int zg_attn_decode(const zg_attn_params* p,
                   const void* q, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, const int* seq_lens,
                   int cache_cap, int ring, const void* gate,
                   const float* q_norm_w, const float* k_norm_w,
                   void* out, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- decode without allocation ------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and semantics as zg_attn_decode without the
 * workspace, and for equal inputs and num_splits the same output and cache
 * bits.  The split partials live in a static device array of
 * ZG_DECODE_NOALLOC_SCRATCH_BYTES per GPU, which the library holds until the
 * process ends; a call whose partials (zg_attn_decode_workspace_size) would
 * not fit returns ZG_ERR_TOO_LARGE before any HIP call.  The array is that
 * of the device current on the calling thread, which must be the stream's
 * device; its address is looked up once per device, on the first call
 * there.  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (two streams, or two threads) race and must be serialised by
 * the caller.  Nothing is allocated; no result depends on the array's
 * previous contents. */
#define ZG_DECODE_NOALLOC_SCRATCH_BYTES (8u << 20)
int zg_attn_decode_noalloc(const zg_attn_params* p,
                           const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int* seq_lens,
                           int cache_cap, int ring, const void* gate,
                           const float* q_norm_w, const float* k_norm_w,
                           void* out, int num_splits, void* stream);

/* Paged KV cache (a serving layout for the global layers' cache, whose size
 * at 256K tokens the structured-data table of the ZGCM-1 page, row
 * "256K 上下文推理 KV 缓存", quantifies): a pool of num_pages pages, each
 * bf16 [Hkv, page_size, D] for K' and the same for V, so k_pages/v_pages are
 * bf16 [num_pages, Hkv, page_size, D].  block_table is device int32
 * [B, max_pages]: token slot t of sequence b lives in page
 * block_table[b*max_pages + t/page_size], row t % page_size.
 *   page_size   a power of two in [32, 65536]
 *   max_pages   table entries per sequence (>= 1); max_pages * page_size
 *               is the per-sequence capacity and must fit an int
 * Table entries are read on the device; an entry outside [0, num_pages) is
 * clamped into that range (the result is then meaningless, but no access
 * leaves the pool).  Pages shared by several sequences are allowed for
 * reading; two sequences must not append into the same page slot. */

/* Copy a prefill's K' (zg_attn_fwd's k_out) and V, both bf16 [B,S,Hkv,D]
 * with B = p->batch and S = p->seqlen, into the page pool: token s of
 * sequence b goes to slot s.  S <= max_pages * page_size is required.
 * S == 0 or B == 0 is valid and launches nothing. */
int zg_attn_kv_write_pages(const zg_attn_params* p,
                           const void* k_prime, const void* v,
                           void* k_pages, void* v_pages, int num_pages,
                           const int* block_table, int max_pages, int page_size,
                           void* stream);

/* zg_attn_decode over a paged cache: identical arguments and semantics to
 * the ring == 0 case of zg_attn_decode with cache_cap = max_pages *
 * page_size, except that key slot t is read from (and the new token's K' and
 * V written to) its page as described above.  The workspace is
 * zg_attn_decode_workspace_size(p, max_pages * page_size, num_splits).  For
 * equal inputs the output is bit-identical to zg_attn_decode's. */
int zg_attn_decode_paged(const zg_attn_params* p,
                         const void* q, const void* k_new, const void* v_new,
                         void* k_pages, void* v_pages, int num_pages,
                         const int* block_table, int max_pages, int page_size,
                         const int* seq_lens, const void* gate,
                         const float* q_norm_w, const float* k_norm_w,
                         void* out, int num_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- One decode step of a block of layers ------------------------------------
 * Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 前置知识 ›
 * 滑动窗口注意力(SWA)与混合注意力 (the model repeats a block of five gated
 * sliding-window layers and one global layer) and the structured-data
 * table, row "256K 上下文推理 KV 缓存" (decode streams the caches).  One
 * launch appends the new token and attends for every layer of such a block:
 * layer l gives the same result as zg_attn_decode with p->window set to
 * layers[l].window, its tensors, the same seq_lens and num_splits =
 * zg_attn_decode_block_num_splits(p, layers[l].cache_cap), bit for bit,
 * including the appended cache rows.  A layer with several splits merges
 * them inside the launch: the last of its workgroups for each (sequence, kv
 * head) to finish combines the partials.
 *
 * bf16 contiguous caches only.  Layers must not share caches or outputs.
 * p->window is ignored (each layer brings its own); every other field of p
 * applies to all layers.  The workspace's ticket words must be zero before
 * the first step (fill a new workspace with zeros); each step leaves them
 * zero again, so the same workspace serves every later step, including
 * replays of a captured graph.  Steps that overlap on one workspace race. */
#define ZG_DECODE_BLOCK_MAX_LAYERS 6
typedef struct zg_decode_layer {
  const void* q;         /* bf16 [B,Hq,D] raw new-token queries */
  const void* k_new;     /* bf16 [B,Hkv,D] raw new key, or NULL (with v_new NULL) */
  const void* v_new;     /* bf16 [B,Hkv,D] */
  void* k_cache;         /* bf16 [B,Hkv,cache_cap,D], updated in place */
  void* v_cache;         /* bf16 [B,Hkv,cache_cap,D], updated in place */
  const void* gate;      /* bf16 [B,Hq,D] or NULL */
  const float* q_norm_w; /* fp32 [D] */
  const float* k_norm_w; /* fp32 [D] */
  void* out;             /* bf16 [B,Hq,D] */
  int cache_cap;         /* >= 1 */
  int ring;              /* 1: ring of cache_cap slots (then window == cache_cap) */
  int window;            /* 0 global, else the band */
} zg_decode_layer;

/* The split count zg_attn_decode_block uses for a layer of this cache
 * capacity (enough splits for one workgroup per CU from that layer alone,
 * at least 256 keys each); 0 if p is invalid or cache_cap < 1. */
int zg_attn_decode_block_num_splits(const zg_attn_params* p, int cache_cap);

/* Bytes of workspace for zg_attn_decode_block (at least 256); 0 if the
 * arguments are invalid.  The workspace itself must be 256-byte aligned. */
size_t zg_attn_decode_block_workspace_size(const zg_attn_params* p, int n_layers,
                                           const zg_decode_layer* layers);
/* 1 <= n_layers <= ZG_DECODE_BLOCK_MAX_LAYERS; seq_lens int32 [B] on the
 * device (clamped as in zg_attn_decode).  Errors as zg_attn_decode's, all
 * reported before the launch. */
int zg_attn_decode_block(const zg_attn_params* p, int n_layers, const zg_decode_layer* layers,
                         const int* seq_lens, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- FP8 (E4M3) KV cache ----------------------------------------------------
 * Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 前置知识 ›
 * FP8 混合精度训练与 TWEO: E4M3 with per-tensor scaling factors is the
 * model's matrix-multiply precision; the page's structured-data table, row
 * "256K 上下文推理 KV 缓存", frames decode cost as the bytes of the cache.
 * Here the cache holds one byte per element: the OCP E4M3 code (bias 7,
 * largest finite 448, 0x7F/0xFF NaN) of K' * k_scale and of V * v_scale,
 * with the product formed in fp32, clamped to [-448, 448] and rounded to
 * the nearest E4M3 value, ties to even (the codes zg_quantize_fp8 writes).
 * A cached key then stands for decode(code) / k_scale and a value for
 * decode(code) / v_scale.  QK^T is an E4M3 product on the FP8 matrix cores:
 * each query head's normalised, rotated row q' is quantized to E4M3 with the
 * power-of-two scale s_q = 2^(8 - e), where amax|q'| = m 2^e, m in [0.5, 1)
 * and e >= -100 (so amax * s_q lies in [128, 256)), and the scores are the
 * fp32 sums of exact code products times 1 / (s_q k_scale).  The softmax is
 * fp32; PV runs on the bf16 matrix cores with each value code widened to
 * bf16 (exact: every E4M3 value is a bf16 value) and P rounded to bf16, and
 * 1 / v_scale is applied to the output.  A step reads half the bytes of a
 * bf16 cache.
 * Scales must be finite and > 0 (else ZG_ERR_INVALID). */

/* zg_attn_decode with uint8 caches k_cache / v_cache [B,Hkv,cache_cap,D] of
 * E4M3 codes; the new token's K' and V are quantized with k_scale / v_scale
 * into their slot (updated in place).  Every other argument, the workspace
 * and the clamping of seq_lens are as for zg_attn_decode. */
int zg_attn_decode_fp8(const zg_attn_params* p,
                       const void* q, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const int* seq_lens,
                       int cache_cap, int ring, float k_scale, float v_scale,
                       const void* gate, const float* q_norm_w, const float* k_norm_w,
                       void* out, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream);

/* zg_attn_decode_paged over uint8 page pools [num_pages,Hkv,page_size,D] of
 * E4M3 codes (scales as for zg_attn_decode_fp8).  For equal inputs the
 * output is bit-identical to zg_attn_decode_fp8's with ring == 0. */
int zg_attn_decode_paged_fp8(const zg_attn_params* p,
                             const void* q, const void* k_new, const void* v_new,
                             void* k_pages, void* v_pages, int num_pages,
                             const int* block_table, int max_pages, int page_size,
                             const int* seq_lens, float k_scale, float v_scale,
                             const void* gate, const float* q_norm_w, const float* k_norm_w,
                             void* out, int num_splits,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- FP8 (E4M3) prefill -------------------------------------------------------
 * The same page and section (E4M3 forward matrix multiplies with per-tensor
 * scaling).  The forward of a global layer (window 0, or a window >= seqlen)
 * with S = K' Q'^T on the FP8 matrix cores: the key prologue writes K' as
 * the E4M3 codes of K' * k_scale (fp32 product, clamp to +-448, round to
 * nearest even; k_scale is the caller's per-tensor scale, finite and > 0),
 * each query head's row q' is quantized with its own power-of-two scale
 * exactly as in zg_attn_decode_fp8, and the scores are the fp32 sums of the
 * exact code products times softmax_scale / (s_q k_scale).  The softmax is
 * fp32 and P V runs on the bf16 matrix cores with V as given, as in
 * zg_attn_fwd.  K' * k_scale should stay well inside +-448: |K'| is at most
 * sqrt(head_dim) max|k_norm_w| per element, so k_scale <= 448 / (11.4
 * max|k_norm_w|) never clamps.
 *
 * Arguments as for zg_attn_fwd, except: k_scale; k_out, when not NULL,
 * receives the uint8 codes [B,S,Hkv,D] (else the workspace holds them, of
 * zg_attn_fwd_fp8_workspace_size bytes, the 256 bytes of queue counters
 * included; with k_out the workspace holds only the counters, 256 bytes).
 * A window in (0, seqlen) returns
 * ZG_ERR_UNSUPPORTED: windowed layers are bound by HBM bytes, which an E4M3
 * score product does not reduce. */
size_t zg_attn_fwd_fp8_workspace_size(const zg_attn_params* p);
int zg_attn_fwd_fp8(const zg_attn_params* p, const void* q, const void* k, const void* v,
                    const void* gate, const float* q_norm_w, const float* k_norm_w,
                    float k_scale, void* out, float* lse, void* k_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---- The projections on either side of the attention ----------------------
 * Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 核心方法, and
 * page "7B 打 235B？…", section 🏗️ 架构: hidden size 4096 feeding 32 query
 * and 8 KV heads of 128 dims; the sliding-window output is multiplied by a
 * sigmoid gate of its own shape, whose logits come from the layer input
 * (reading: a linear projection, since the gate's formula did not survive
 * on the page).  Weights are stored [out_features, in_features] (a bias-free
 * linear map y = x W^T); bf16 operands and results, fp32 accumulation.
 * Neither call allocates or needs a workspace. */

/* y bf16 [M,N] = x bf16 [M,K] . w bf16 [N,K]^T (the output projection is
 * M = tokens, N = hidden, K = n_q_heads * head_dim).  N must be a multiple of
 * 256 and K a positive multiple of 32 (else ZG_ERR_UNSUPPORTED); M is any
 * size >= 0.  M == 0 or N == 0 is valid and launches nothing. */
int zg_linear(int M, int N, int K, const void* x, const void* w, void* y, void* stream);

/* The fused input projection of one layer for T = p->batch * p->seqlen
 * tokens: x bf16 [T,hidden]; w bf16 [Nw,hidden] stacking W_q (Hq*D rows),
 * W_k and W_v (Hkv*D rows each) and, when gate != NULL, W_g (Hq*D rows), so
 * Nw = 2*Hkv*D + Hq*D (+ Hq*D).  One GEMM writes q bf16 [T,Hq,D], k and v
 * bf16 [T,Hkv,D] and gate bf16 [T,Hq,D]: the layouts zg_attn_fwd reads.
 * Requires Hkv*D a multiple of 256 (even n_kv_heads) and hidden a positive
 * multiple of 32 (else ZG_ERR_UNSUPPORTED). */
int zg_qkvg_proj(const zg_attn_params* p, int hidden, const void* x, const void* w,
                 void* q, void* k, void* v, void* gate, void* stream);

/* ---- FP8 (E4M3) projections ------------------------------------------------
 * Page "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型", section 前置知识 ›
 * FP8 混合精度训练与 TWEO: the forward matrix multiplies run in 8-bit floating
 * point E4M3 with per-tensor scaling factors (the pages update them from the
 * maximum seen over the last 1024 steps; choosing the factor is the
 * caller's).  E4M3 here is the OCP format: bias 7, no infinities, largest
 * finite value 448. */

/* q uint8 [n] = E4M3 code of x * scale for x bf16 [n]: the product is taken
 * in fp32, clamped to [-448, 448] and rounded to nearest, ties to even (so
 * a value that would overflow saturates).  n a multiple of 8 (else
 * ZG_ERR_UNSUPPORTED); scale finite and > 0; x 16-byte and q 8-byte
 * aligned. */
int zg_quantize_fp8(long long n, const void* x, float scale, void* q, void* stream);

/* y bf16 [M,N] = out_scale * (xq [M,K] . wq [N,K]^T) for E4M3 operands
 * (quantized with scales s_x and s_w, pass out_scale = 1 / (s_x s_w)); the
 * exact products are accumulated in fp32 on the gfx950 FP8 matrix cores
 * (twice the bf16 rate) and the scaled sum is rounded once to bf16.  N a
 * multiple of 256 and K a positive multiple of 128 (else
 * ZG_ERR_UNSUPPORTED); M any size >= 0. */
int zg_linear_fp8(int M, int N, int K, const void* xq, const void* wq, float out_scale,
                  void* y, void* stream);

/* Bytes of device workspace zg_attn_bwd needs (recomputed Q' * c and K',
 * dO, per-row -LSE*log2(e) and rowsum(dY*Y), one partial sum of a weight
 * gradient per workgroup of the two attention-gradient kernels, and 256
 * chunk sums of each); 0 for an invalid p. */
size_t zg_attn_bwd_workspace_size(const zg_attn_params* p);

/* Training backward of one attention layer: the gradients of
 * L = sum(dout * out) for out = zg_attn_fwd(...) with the same p and inputs.
 * The pages define only the forward; this is its derivative by the chain
 * rule (gate, softmax attention, RoPE rotation transposed, RMSNorm).
 *   q, k, v, gate, q_norm_w, k_norm_w   the forward's inputs (gate may be NULL)
 *   out   bf16 [B,S,Hq,D]  the forward's output (gated)
 *   lse   fp32 [B,Hq,S]    the forward's LSE (required)
 *   dout  bf16 [B,S,Hq,D]  dL/dout
 *   dq    bf16 [B,S,Hq,D], dk, dv bf16 [B,S,Hkv,D]   gradients of q, k, v
 *   dgate bf16 [B,S,Hq,D]  gradient of the gate logits; required iff gate
 *   dq_norm_w, dk_norm_w  fp32 [D] weight gradients (overwritten, not
 *         accumulated)
 * dq, dk, dv, dgate and the weight gradients are written in full; the
 * summation order is fixed, so repeated calls give identical bits.
 * S == 0 or B == 0 is valid and launches nothing (the weight-gradient
 * buffers are then left as they are; the gradient is zero). */
int zg_attn_bwd(const zg_attn_params* p,
                const void* q, const void* k, const void* v, const void* gate,
                const float* q_norm_w, const float* k_norm_w,
                const void* out, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, void* dgate,
                float* dq_norm_w, float* dk_norm_w,
                void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* zg_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ZG_ATTN_H */
