// C ABI of libzgattn (declared in include/zg_attn.h): argument validation,
// workspace sizing and kernel launches on the caller's stream.
//
// Nothing here allocates device memory or synchronises; every error is
// reported before the first launch.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/zg_attn.h"
#include "zg_launch.h"

namespace {

using zg::kD;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Shape / numeric checks common to both entry points.
int check_params(const zg_attn_params* p) {
  if (!p) return ZG_ERR_INVALID;
  if (p->batch < 0 || p->seqlen < 0 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->window < 0)
    return ZG_ERR_INVALID;
  if (p->n_q_heads % p->n_kv_heads != 0) return ZG_ERR_INVALID;
  const int grp = p->n_q_heads / p->n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return ZG_ERR_UNSUPPORTED;
  if (p->head_dim <= 0) return ZG_ERR_INVALID;
  if (p->head_dim != kD) return ZG_ERR_UNSUPPORTED;
  if (p->rope_dim < 0 || (p->rope_dim & 1) || p->rope_dim > p->head_dim) return ZG_ERR_INVALID;
  if (p->rope_dim > p->head_dim / 2) return ZG_ERR_UNSUPPORTED;
  if (p->rope_dim > 0 && !(isfinite(p->rope_theta) && p->rope_theta > 0.f)) return ZG_ERR_INVALID;
  if (!(isfinite(p->rms_eps) && p->rms_eps >= 0.f)) return ZG_ERR_INVALID;
  if (!(isfinite(p->softmax_scale) && p->softmax_scale >= 0.f)) return ZG_ERR_INVALID;
  return ZG_OK;
}

zg::RopeTable make_rope_table(const zg_attn_params* p) {
  zg::RopeTable t{};
  const int half = p->rope_dim / 2;
  const long double two_pi = 2.0L * acosl(-1.0L);
  for (int i = 0; i < half; ++i) {
    // revolutions per position, < 1/(2 pi), as a 0.64 fixed-point fraction
    const long double rev = powl((long double)p->rope_theta, -2.0L * i / (long double)p->rope_dim) / two_pi;
    t.frac[i] = (uint64_t)(ldexpl(rev, 64) + 0.5L);
  }
  return t;
}

float scale_log2(const zg_attn_params* p) {
  const double s = p->softmax_scale > 0.f ? (double)p->softmax_scale : 1.0 / sqrt((double)kD);
  return (float)(s * 1.4426950408889634);
}

int hip_status(hipError_t e) { return e == hipSuccess ? ZG_OK : ZG_ERR_HIP; }

// The no-allocation decode's split partials: one array per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// a device address; the address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is passed to kernels.
constexpr size_t kNoallocScratchBytes = ZG_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on first use).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ZG_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ZG_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ZG_OK;
}

size_t kprime_bytes(const zg_attn_params* p) {
  return (size_t)p->batch * (size_t)p->seqlen * (size_t)p->n_kv_heads * kD * 2;
}

int auto_splits(const zg_attn_params* p, int cache_cap) {
  const long long pairs = (long long)p->batch * p->n_kv_heads;
  if (pairs <= 0) return 1;
  long long s = (1024 + pairs - 1) / pairs;       // ~4 workgroups per CU
  const long long by_len = (cache_cap + 255) / 256;  // >= 256 keys per split
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

// Backward workspace: 256-byte aligned segments, in this order.
struct BwdLayout {
  size_t qp, kp, dO, lse2, dvec, part_q, part_k, red, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The causal kernel's 16 work-queue counters, at the end of the forward
// workspace.
constexpr size_t kQueueBytes = 256;

BwdLayout bwd_layout(const zg_attn_params* p) {
  const size_t B = (size_t)p->batch, S = (size_t)p->seqlen, Hq = (size_t)p->n_q_heads,
               Hkv = (size_t)p->n_kv_heads;
  const size_t Spad = (S + zg::kBwdRowPad - 1) / zg::kBwdRowPad * zg::kBwdRowPad;
  BwdLayout l;
  size_t off = 0;
  l.qp = off;   off += align256(B * S * Hq * kD * 2);
  l.kp = off;   off += align256(B * S * Hkv * kD * 2);
  l.dO = off;   off += align256(B * S * Hq * kD * 2);
  l.lse2 = off; off += align256(B * Hq * Spad * 4);
  l.dvec = off; off += align256(B * Hq * Spad * 4);
  l.part_q = off;
  off += align256((size_t)zg::bwd_dq_blocks((int)B, (int)S, (int)Hq, (int)Hkv) * kD * 4);
  l.part_k = off;
  off += align256((size_t)zg::bwd_dkv_blocks((int)B, (int)S, (int)Hkv) * kD * 4);
  l.red = off;  off += align256((size_t)2 * zg::kBwdRedChunks * kD * 4);
  l.total = off;
  return l;
}

}  // namespace

// Shared body of the fixed-length and the packed forward.  `total` rows of
// the token-major tensors; cu_seqlens null means B sequences of S rows.
static int fwd_impl(const zg_attn_params* p, const int* cu_seqlens, long long total,
                    const void* q, const void* k, const void* v, const void* gate,
                    const float* q_norm_w, const float* k_norm_w, void* out, float* lse,
                    void* k_out, void* workspace, size_t workspace_bytes, void* stream) {
  if ((long long)p->seqlen * p->n_q_heads > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (p->batch == 0 || p->seqlen == 0) return ZG_OK;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !out) return ZG_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || !aligned16(out) || (gate && !aligned16(gate)) ||
      (k_out && !aligned16(k_out)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ZG_ERR_INVALID;
  const size_t kp_bytes = (size_t)total * (size_t)p->n_kv_heads * kD * 2;
  const bool causal = p->window == 0;
  void* kp = k_out;
  int* queue = nullptr;
  if (!kp || causal) {
    // K' (without k_out), then the causal kernel's queue counters
    const size_t need = (kp ? 0 : align256(kp_bytes)) + (causal ? kQueueBytes : 0);
    if (!workspace || workspace_bytes < need) return ZG_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ZG_ERR_INVALID;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if (!kp) kp = ws;
    if (causal) queue = reinterpret_cast<int*>(ws + need - kQueueBytes);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const zg::RopeTable tab = make_rope_table(p);
  const long long krows = total * p->n_kv_heads;
  hipError_t e = zg::launch_k_prologue(static_cast<const uint16_t*>(k), k_norm_w,
                                       static_cast<uint16_t*>(kp), krows, p->seqlen,
                                       p->n_kv_heads, p->pos_offset, p->rope_dim / 2,
                                       p->rms_eps, tab, s, cu_seqlens, p->batch, 1.0f, queue);
  if (e != hipSuccess) return ZG_ERR_HIP;
  zg::FlashParams fp{};
  fp.q = static_cast<const uint16_t*>(q);
  fp.kp = static_cast<const uint16_t*>(kp);
  fp.v = static_cast<const uint16_t*>(v);
  fp.gate = static_cast<const uint16_t*>(gate);
  fp.q_norm_w = q_norm_w;
  fp.k_norm_w = k_norm_w;
  fp.out = static_cast<uint16_t*>(out);
  fp.lse = lse;
  fp.cu_seqlens = cu_seqlens;
  fp.total = total;
  fp.B = p->batch;
  fp.S = p->seqlen;
  fp.Hq = p->n_q_heads;
  fp.Hkv = p->n_kv_heads;
  fp.window = p->window;
  fp.rope_half = p->rope_dim / 2;
  fp.scale_log2 = scale_log2(p);
  fp.eps = p->rms_eps;
  fp.pos_offset = p->pos_offset;
  fp.tab = tab;
  fp.queue = queue;
  return hip_status(zg::launch_flash_fwd(fp, s));
}

// The E4M3 forward of a global layer (fixed-length batches).
static int fwd_fp8_impl(const zg_attn_params* p, const void* q, const void* k, const void* v,
                        const void* gate, const float* q_norm_w, const float* k_norm_w,
                        float k_scale, void* out, float* lse, void* k_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!(isfinite(k_scale) && k_scale > 0.f)) return ZG_ERR_INVALID;
  if (p->window > 0 && p->window < p->seqlen) return ZG_ERR_UNSUPPORTED;
  if ((long long)p->seqlen * p->n_q_heads > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (p->batch == 0 || p->seqlen == 0) return ZG_OK;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !out) return ZG_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || !aligned16(out) || (gate && !aligned16(gate)) ||
      (k_out && !aligned16(k_out)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ZG_ERR_INVALID;
  // workspace: the K' codes (without k_out), then the queue counters
  void* kp = k_out;
  const size_t need = (kp ? 0 : align256(kprime_bytes(p) / 2)) + kQueueBytes;
  if (!workspace || workspace_bytes < need) return ZG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ZG_ERR_INVALID;
  if (!kp) kp = workspace;
  int* queue = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + need - kQueueBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const zg::RopeTable tab = make_rope_table(p);
  hipError_t e = zg::launch_k_prologue_fp8(
      static_cast<const uint16_t*>(k), k_norm_w, static_cast<uint8_t*>(kp), k_scale,
      (long long)p->batch * p->seqlen * p->n_kv_heads, p->seqlen, p->n_kv_heads, p->pos_offset,
      p->rope_dim / 2, p->rms_eps, tab, s, nullptr, 0, queue);
  if (e != hipSuccess) return ZG_ERR_HIP;
  zg::FlashParams fp{};
  fp.q = static_cast<const uint16_t*>(q);
  fp.kp8 = static_cast<const uint8_t*>(kp);
  fp.k_scale = k_scale;
  fp.v = static_cast<const uint16_t*>(v);
  fp.gate = static_cast<const uint16_t*>(gate);
  fp.q_norm_w = q_norm_w;
  fp.k_norm_w = k_norm_w;
  fp.out = static_cast<uint16_t*>(out);
  fp.lse = lse;
  fp.total = (long long)p->batch * p->seqlen;
  fp.B = p->batch;
  fp.S = p->seqlen;
  fp.Hq = p->n_q_heads;
  fp.Hkv = p->n_kv_heads;
  fp.window = 0;
  fp.rope_half = p->rope_dim / 2;
  fp.scale_log2 = scale_log2(p);
  fp.eps = p->rms_eps;
  fp.pos_offset = p->pos_offset;
  fp.tab = tab;
  fp.queue = queue;
  return hip_status(zg::launch_flash_causal(fp, s));
}

// Shared body of the contiguous and the paged decode.
static int decode_impl(const zg_attn_params* p, const void* q, const void* k_new,
                       const void* v_new, void* k_cache, void* v_cache, const int* seq_lens,
                       int cache_cap, int ring, const zg::CacheMap& map, const void* gate,
                       const float* q_norm_w, const float* k_norm_w, void* out, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream, int fp8 = 0,
                       float k_scale = 0.f, float v_scale = 0.f) {
  int st = check_params(p);
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return ZG_ERR_INVALID;
  if (st != ZG_OK) return st;
  if (cache_cap < 1 || num_splits < 0 || num_splits > 256) return ZG_ERR_INVALID;
  if (ring && p->window != cache_cap) return ZG_ERR_INVALID;
  if ((k_new == nullptr) != (v_new == nullptr)) return ZG_ERR_INVALID;
  if (p->batch == 0) return ZG_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !q_norm_w || !k_norm_w || !out)
    return ZG_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || !aligned16(out) || (gate && !aligned16(gate)) ||
      (k_new && (!aligned16(k_new) || !aligned16(v_new))) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return ZG_ERR_INVALID;
  const int ns = num_splits ? num_splits : auto_splits(p, cache_cap);
  const size_t need = (size_t)p->batch * p->n_q_heads * ns * (kD + 2) * sizeof(float);
  if (!workspace || workspace_bytes < need) return ZG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ZG_ERR_INVALID;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const zg::RopeTable tab = make_rope_table(p);
  zg::DecodeParams dp{};
  if (k_new && ns == 1) {  // the single-split kernel appends the token itself
    dp.k_new = static_cast<const uint16_t*>(k_new);
    dp.v_new = static_cast<const uint16_t*>(v_new);
    dp.k_norm_w = k_norm_w;
  } else if (k_new) {
    hipError_t e = zg::launch_decode_append(
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), k_cache,
        v_cache, seq_lens, k_norm_w, p->batch, p->n_kv_heads, cache_cap, ring, map,
        p->pos_offset, p->rope_dim / 2, p->rms_eps, tab, fp8, k_scale, v_scale, s);
    if (e != hipSuccess) return ZG_ERR_HIP;
  }
  dp.q = static_cast<const uint16_t*>(q);
  dp.k_cache = static_cast<const uint16_t*>(k_cache);
  dp.v_cache = static_cast<const uint16_t*>(v_cache);
  dp.seq_lens = seq_lens;
  dp.q_norm_w = q_norm_w;
  dp.gate = static_cast<const uint16_t*>(gate);
  dp.out = static_cast<uint16_t*>(out);
  float* ws = static_cast<float*>(workspace);
  dp.part_o = ws;
  dp.part_ml = ws + (size_t)p->batch * p->n_q_heads * ns * kD;
  dp.B = p->batch;
  dp.Hq = p->n_q_heads;
  dp.Hkv = p->n_kv_heads;
  dp.cap = cache_cap;
  dp.ring = ring;
  dp.window = p->window;
  dp.nsplit = ns;
  dp.rope_half = p->rope_dim / 2;
  dp.scale_log2 = scale_log2(p);
  dp.eps = p->rms_eps;
  dp.pos_offset = p->pos_offset;
  dp.map = map;
  dp.tab = tab;
  if (fp8) {
    // scores are q'.decode(code) / k_scale: fold the division into the scale
    dp.fp8 = 1;
    dp.k_scale = k_scale;
    dp.v_scale = v_scale;
    dp.scale_log2 = (float)((double)dp.scale_log2 / (double)k_scale);
    dp.v_inv = (float)(1.0 / (double)v_scale);
  }
  return hip_status(zg::launch_decode(dp, s));
}

static_assert(zg::kMaxBlockLayers == ZG_DECODE_BLOCK_MAX_LAYERS, "block layer limit");

// Workspace of a block decode step: the ticket words of every layer with
// several splits (one uint32 per (b, kv head)), then those layers' partials
// ([B,Hq,ns,D] fp32 followed by [B,Hq,ns,2]), in 256-byte aligned segments.
struct BlockLayout {
  int ns[zg::kMaxBlockLayers];
  size_t tickets[zg::kMaxBlockLayers];
  size_t part[zg::kMaxBlockLayers];
  size_t total;
};

// Splits of one layer in a block decode step: enough that the layer alone
// has a workgroup per CU (256), each split at least 256 keys.  The block's
// other layers fill the remaining slots, so fewer, longer splits than a
// one-layer decode's (auto_splits) pay less per-workgroup overhead.
static int block_splits(const zg_attn_params* p, int cache_cap) {
  const long long pairs = (long long)p->batch * p->n_kv_heads;
  if (pairs <= 0) return 1;
  long long s = (256 + pairs - 1) / pairs;
  const long long by_len = (cache_cap + 255) / 256;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

static int block_layout(const zg_attn_params* p, int n_layers, const zg_decode_layer* layers,
                        BlockLayout& lay) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  if (n_layers < 1 || n_layers > ZG_DECODE_BLOCK_MAX_LAYERS || !layers) return ZG_ERR_INVALID;
  size_t off = 0;
  for (int l = 0; l < n_layers; ++l) {
    const zg_decode_layer& L = layers[l];
    if (L.cache_cap < 1 || (L.ring != 0 && L.ring != 1) || L.window < 0) return ZG_ERR_INVALID;
    if (L.ring && L.window != L.cache_cap) return ZG_ERR_INVALID;
    lay.ns[l] = block_splits(p, L.cache_cap);
    lay.tickets[l] = 0;
    if (lay.ns[l] > 1) {
      lay.tickets[l] = off;
      off += align256((size_t)p->batch * p->n_kv_heads * sizeof(unsigned));
    }
  }
  for (int l = 0; l < n_layers; ++l) {
    lay.part[l] = 0;
    if (lay.ns[l] > 1) {
      lay.part[l] = off;
      off += align256((size_t)p->batch * p->n_q_heads * lay.ns[l] * (kD + 2) * sizeof(float));
    }
  }
  lay.total = off;
  return ZG_OK;
}

// Page-pool arguments: page_size a power of two in [32, 65536], a table of
// max_pages >= 1 entries per sequence, at least one page, and a slot count
// (max_pages * page_size) that fits an int.
static int check_pages(int num_pages, const int* block_table, int max_pages, int page_size,
                       zg::CacheMap& map) {
  if (num_pages < 1 || !block_table || max_pages < 1) return ZG_ERR_INVALID;
  if (page_size < 32 || page_size > 65536 || (page_size & (page_size - 1))) return ZG_ERR_INVALID;
  if ((long long)max_pages * page_size > 0x7fffffffLL) return ZG_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return ZG_ERR_INVALID;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  map = zg::CacheMap{block_table, max_pages, sh, num_pages};
  return ZG_OK;
}

extern "C" {

const char* zg_attn_strerror(int status) {
  switch (status) {
    case ZG_OK: return "ok";
    case ZG_ERR_INVALID: return "invalid argument (null pointer, bad shape or misaligned pointer)";
    case ZG_ERR_UNSUPPORTED: return "unsupported configuration";
    case ZG_ERR_WORKSPACE: return "workspace missing or too small";
    case ZG_ERR_HIP: return "HIP launch or runtime error";
    case ZG_ERR_TOO_LARGE:
      return "the split partials exceed the no-allocation decode's static scratch";
    default: return "unknown status";
  }
}

size_t zg_attn_fwd_workspace_size(const zg_attn_params* p) {
  if (check_params(p) != ZG_OK) return 0;
  if (kprime_bytes(p) == 0) return 0;  // nothing is launched
  return align256(kprime_bytes(p)) + (p->window == 0 ? kQueueBytes : 0);
}

int zg_attn_fwd(const zg_attn_params* p, const void* q, const void* k, const void* v,
                const void* gate, const float* q_norm_w, const float* k_norm_w, void* out,
                float* lse, void* k_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  return fwd_impl(p, nullptr, (long long)p->batch * p->seqlen, q, k, v, gate, q_norm_w,
                  k_norm_w, out, lse, k_out, workspace, workspace_bytes, stream);
}

size_t zg_attn_fwd_varlen_workspace_size(const zg_attn_params* p, long long total_tokens) {
  if (check_params(p) != ZG_OK || total_tokens < 0) return 0;
  if (total_tokens == 0 || p->batch == 0 || p->seqlen == 0) return 0;  // nothing is launched
  return align256((size_t)total_tokens * (size_t)p->n_kv_heads * kD * 2) +
         (p->window == 0 ? kQueueBytes : 0);
}

int zg_attn_fwd_varlen(const zg_attn_params* p, const int* cu_seqlens, long long total_tokens,
                       const void* q, const void* k, const void* v, const void* gate,
                       const float* q_norm_w, const float* k_norm_w, void* out, float* lse,
                       void* k_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  if (total_tokens < 0) return ZG_ERR_INVALID;
  if (p->batch > 0 && (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)))
    return ZG_ERR_INVALID;
  if (p->batch == 0 || p->seqlen == 0 || total_tokens == 0) return ZG_OK;
  return fwd_impl(p, cu_seqlens, total_tokens, q, k, v, gate, q_norm_w, k_norm_w, out, lse,
                  k_out, workspace, workspace_bytes, stream);
}

size_t zg_attn_fwd_fp8_workspace_size(const zg_attn_params* p) {
  if (check_params(p) != ZG_OK) return 0;
  if (kprime_bytes(p) == 0) return 0;  // nothing is launched
  return align256(kprime_bytes(p) / 2) + kQueueBytes;
}

int zg_attn_fwd_fp8(const zg_attn_params* p, const void* q, const void* k, const void* v,
                    const void* gate, const float* q_norm_w, const float* k_norm_w,
                    float k_scale, void* out, float* lse, void* k_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  return fwd_fp8_impl(p, q, k, v, gate, q_norm_w, k_norm_w, k_scale, out, lse, k_out, workspace,
                      workspace_bytes, stream);
}

size_t zg_attn_bwd_workspace_size(const zg_attn_params* p) {
  if (check_params(p) != ZG_OK) return 0;
  return bwd_layout(p).total;
}

int zg_attn_bwd(const zg_attn_params* p, const void* q, const void* k, const void* v,
                const void* gate, const float* q_norm_w, const float* k_norm_w, const void* out,
                const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dgate,
                float* dq_norm_w, float* dk_norm_w, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  if ((long long)p->seqlen * p->n_q_heads > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (p->batch == 0 || p->seqlen == 0) return ZG_OK;
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !out || !lse || !dout || !dq || !dk || !dv ||
      !dq_norm_w || !dk_norm_w)
    return ZG_ERR_INVALID;
  if ((gate == nullptr) != (dgate == nullptr)) return ZG_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (gate && (!aligned16(gate) || !aligned16(dgate))) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(dq_norm_w) & 3u) ||
      (reinterpret_cast<uintptr_t>(dk_norm_w) & 3u))
    return ZG_ERR_INVALID;
  const BwdLayout L = bwd_layout(p);
  if (!workspace || workspace_bytes < L.total) return ZG_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ZG_ERR_INVALID;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* qp = reinterpret_cast<uint16_t*>(ws + L.qp);
  uint16_t* kp = reinterpret_cast<uint16_t*>(ws + L.kp);
  uint16_t* dO = gate ? reinterpret_cast<uint16_t*>(ws + L.dO)
                      : const_cast<uint16_t*>(static_cast<const uint16_t*>(dout));
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  float* dvec = reinterpret_cast<float*>(ws + L.dvec);
  const int B = p->batch, S = p->seqlen, Hq = p->n_q_heads, Hkv = p->n_kv_heads;
  const int Spad = (S + zg::kBwdRowPad - 1) / zg::kBwdRowPad * zg::kBwdRowPad;
  const zg::RopeTable tab = make_rope_table(p);
  const int rh = p->rope_dim / 2;

  // K' is recomputed in the prep launch
  zg::KPrimeJob kj{};
  kj.k = static_cast<const uint16_t*>(k);
  kj.w = k_norm_w;
  kj.kout = kp;
  kj.rows = (long long)B * S * Hkv;
  kj.S = S;
  kj.Hkv = Hkv;
  kj.pos_offset = p->pos_offset;
  kj.rope_half = rh;
  kj.eps = p->rms_eps;
  kj.tab = tab;
  hipError_t e = zg::launch_bwd_prep(static_cast<const uint16_t*>(dout),
                                     static_cast<const uint16_t*>(out),
                                     static_cast<const uint16_t*>(gate), lse, dO,
                                     static_cast<uint16_t*>(dgate), lse2, dvec, B, S, Spad, Hq, kj,
                                     s);
  if (e != hipSuccess) return ZG_ERR_HIP;
  if (!zg::bwd_dq_fuses_q(rh)) {  // else the dq' kernel forms Q' * c itself
    e = zg::launch_k_prologue(static_cast<const uint16_t*>(q), q_norm_w, qp, (long long)B * S * Hq,
                              S, Hq, p->pos_offset, rh, p->rms_eps, tab, s, nullptr, 0,
                              scale_log2(p));
    if (e != hipSuccess) return ZG_ERR_HIP;
  }
  zg::BwdParams bp{};
  bp.qp = qp;
  bp.kp = kp;
  bp.v = static_cast<const uint16_t*>(v);
  bp.dO = dO;
  bp.nlse2 = lse2;
  bp.dvec = dvec;
  bp.dq = static_cast<uint16_t*>(dq);
  bp.dk = static_cast<uint16_t*>(dk);
  bp.part_q = reinterpret_cast<float*>(ws + L.part_q);
  bp.part_k = reinterpret_cast<float*>(ws + L.part_k);
  bp.dv = static_cast<uint16_t*>(dv);
  bp.B = B;
  bp.S = S;
  bp.Spad = Spad;
  bp.Hq = Hq;
  bp.Hkv = Hkv;
  // a window of at least S sees every causal key; clamping keeps the key
  // kernel's band arithmetic (last query of a key block = keys + window - 1)
  // inside int for any window up to INT_MAX
  bp.window = p->window > S ? S : p->window;
  bp.scale_log2 = scale_log2(p);
  bp.scale = (float)(p->softmax_scale > 0.f ? (double)p->softmax_scale : 1.0 / sqrt((double)kD));
  bp.q = static_cast<const uint16_t*>(q);
  bp.k = static_cast<const uint16_t*>(k);
  bp.q_norm_w = q_norm_w;
  bp.k_norm_w = k_norm_w;
  bp.eps = p->rms_eps;
  bp.rope_half = rh;
  bp.pos_offset = p->pos_offset;
  bp.tab = tab;
  if (zg::launch_bwd_dq(bp, s) != hipSuccess) return ZG_ERR_HIP;
  if (zg::launch_bwd_dkv(bp, s) != hipSuccess) return ZG_ERR_HIP;
  return hip_status(zg::launch_reduce_parts(bp, reinterpret_cast<float*>(ws + L.red), dq_norm_w,
                                              dk_norm_w, s));
}

int zg_attn_decode_num_splits(const zg_attn_params* p, int cache_cap) {
  if (check_params(p) != ZG_OK || cache_cap < 1) return 0;
  return auto_splits(p, cache_cap);
}

size_t zg_attn_decode_workspace_size(const zg_attn_params* p, int cache_cap, int num_splits) {
  if (check_params(p) != ZG_OK || cache_cap < 1 || num_splits < 0 || num_splits > 256) return 0;
  const int ns = num_splits ? num_splits : auto_splits(p, cache_cap);
  return (size_t)p->batch * p->n_q_heads * ns * (kD + 2) * sizeof(float);
}

int zg_attn_decode(const zg_attn_params* p, const void* q, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, const int* seq_lens, int cache_cap, int ring,
                   const void* gate, const float* q_norm_w, const float* k_norm_w, void* out,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (ring != 0 && ring != 1) return ZG_ERR_INVALID;
  const zg::CacheMap contiguous{nullptr, 0, 0, 0};
  return decode_impl(p, q, k_new, v_new, k_cache, v_cache, seq_lens, cache_cap, ring, contiguous,
                     gate, q_norm_w, k_norm_w, out, num_splits, workspace, workspace_bytes,
                     stream);
}

int zg_attn_decode_block_num_splits(const zg_attn_params* p, int cache_cap) {
  if (check_params(p) != ZG_OK || cache_cap < 1) return 0;
  return block_splits(p, cache_cap);
}

size_t zg_attn_decode_block_workspace_size(const zg_attn_params* p, int n_layers,
                                           const zg_decode_layer* layers) {
  BlockLayout lay;
  if (block_layout(p, n_layers, layers, lay) != ZG_OK) return 0;
  return lay.total > 256 ? lay.total : 256;
}

int zg_attn_decode_block(const zg_attn_params* p, int n_layers, const zg_decode_layer* layers,
                         const int* seq_lens, void* workspace, size_t workspace_bytes,
                         void* stream) {
  BlockLayout lay;
  int st = block_layout(p, n_layers, layers, lay);
  if (st != ZG_OK) return st;
  if (p->batch == 0) return ZG_OK;
  if (!seq_lens || (reinterpret_cast<uintptr_t>(seq_lens) & 3u)) return ZG_ERR_INVALID;
  for (int l = 0; l < n_layers; ++l) {
    const zg_decode_layer& L = layers[l];
    if ((L.k_new == nullptr) != (L.v_new == nullptr)) return ZG_ERR_INVALID;
    if (!L.q || !L.k_cache || !L.v_cache || !L.q_norm_w || !L.k_norm_w || !L.out)
      return ZG_ERR_INVALID;
    if (!aligned16(L.q) || !aligned16(L.k_cache) || !aligned16(L.v_cache) ||
        !aligned16(L.q_norm_w) || !aligned16(L.k_norm_w) || !aligned16(L.out) ||
        (L.gate && !aligned16(L.gate)) || (L.k_new && (!aligned16(L.k_new) || !aligned16(L.v_new))))
      return ZG_ERR_INVALID;
  }
  if (lay.total > 0) {
    if (!workspace || workspace_bytes < lay.total) return ZG_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return ZG_ERR_INVALID;
  }
  const zg::RopeTable tab = make_rope_table(p);
  zg::DecodeBlockParams bp{};
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  long long wg = 0;
  int slot = 0;
  // layers with several splits (the long ones) are launched first
  for (int pass = 0; pass < 2; ++pass) {
    for (int l = 0; l < n_layers; ++l) {
      if ((lay.ns[l] > 1) != (pass == 0)) continue;
      const zg_decode_layer& L = layers[l];
      zg::DecodeParams& dp = bp.layer[slot];
      dp.q = static_cast<const uint16_t*>(L.q);
      dp.k_new = static_cast<const uint16_t*>(L.k_new);
      dp.v_new = static_cast<const uint16_t*>(L.v_new);
      dp.k_norm_w = L.k_norm_w;
      dp.k_cache = static_cast<const uint16_t*>(L.k_cache);
      dp.v_cache = static_cast<const uint16_t*>(L.v_cache);
      dp.seq_lens = seq_lens;
      dp.q_norm_w = L.q_norm_w;
      dp.gate = static_cast<const uint16_t*>(L.gate);
      dp.out = static_cast<uint16_t*>(L.out);
      dp.B = p->batch;
      dp.Hq = p->n_q_heads;
      dp.Hkv = p->n_kv_heads;
      dp.cap = L.cache_cap;
      dp.ring = L.ring;
      dp.window = L.window;
      dp.nsplit = lay.ns[l];
      dp.rope_half = p->rope_dim / 2;
      dp.scale_log2 = scale_log2(p);
      dp.eps = p->rms_eps;
      dp.pos_offset = p->pos_offset;
      dp.map = zg::CacheMap{nullptr, 0, 0, 0};
      dp.tab = tab;
      if (lay.ns[l] > 1) {
        dp.tickets = reinterpret_cast<unsigned*>(ws + lay.tickets[l]);
        dp.part_o = reinterpret_cast<float*>(ws + lay.part[l]);
        dp.part_ml = dp.part_o + (size_t)p->batch * p->n_q_heads * lay.ns[l] * kD;
      }
      bp.wg0[slot] = (int)wg;
      wg += (long long)p->batch * p->n_kv_heads * lay.ns[l];
      if (wg > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
      ++slot;
    }
  }
  bp.n_layers = n_layers;
  return hip_status(zg::launch_decode_block(bp, (int)wg, reinterpret_cast<hipStream_t>(stream)));
}

int zg_attn_decode_noalloc(const zg_attn_params* p, const void* q, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache, const int* seq_lens,
                           int cache_cap, int ring, const void* gate, const float* q_norm_w,
                           const float* k_norm_w, void* out, int num_splits, void* stream) {
  if (ring != 0 && ring != 1) return ZG_ERR_INVALID;
  const int st = check_params(p);
  if (st != ZG_OK) return st;
  if (cache_cap < 1 || num_splits < 0 || num_splits > 256) return ZG_ERR_INVALID;
  if (p->batch == 0) return ZG_OK;
  // the size check comes before any HIP call
  if (zg_attn_decode_workspace_size(p, cache_cap, num_splits) > kNoallocScratchBytes)
    return ZG_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int sst = noalloc_scratch(&ws);
  if (sst != ZG_OK) return sst;
  const zg::CacheMap contiguous{nullptr, 0, 0, 0};
  return decode_impl(p, q, k_new, v_new, k_cache, v_cache, seq_lens, cache_cap, ring, contiguous,
                     gate, q_norm_w, k_norm_w, out, num_splits, ws, kNoallocScratchBytes, stream);
}

int zg_attn_decode_paged(const zg_attn_params* p, const void* q, const void* k_new,
                         const void* v_new, void* k_pages, void* v_pages, int num_pages,
                         const int* block_table, int max_pages, int page_size,
                         const int* seq_lens, const void* gate, const float* q_norm_w,
                         const float* k_norm_w, void* out, int num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
  zg::CacheMap map{};
  const int st = check_pages(num_pages, block_table, max_pages, page_size, map);
  if (st != ZG_OK) return st;
  return decode_impl(p, q, k_new, v_new, k_pages, v_pages, seq_lens, max_pages * page_size, 0,
                     map, gate, q_norm_w, k_norm_w, out, num_splits, workspace, workspace_bytes,
                     stream);
}

int zg_attn_decode_fp8(const zg_attn_params* p, const void* q, const void* k_new,
                       const void* v_new, void* k_cache, void* v_cache, const int* seq_lens,
                       int cache_cap, int ring, float k_scale, float v_scale, const void* gate,
                       const float* q_norm_w, const float* k_norm_w, void* out, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const zg::CacheMap contiguous{nullptr, 0, 0, 0};
  return decode_impl(p, q, k_new, v_new, k_cache, v_cache, seq_lens, cache_cap, ring, contiguous,
                     gate, q_norm_w, k_norm_w, out, num_splits, workspace, workspace_bytes,
                     stream, 1, k_scale, v_scale);
}

int zg_attn_decode_paged_fp8(const zg_attn_params* p, const void* q, const void* k_new,
                             const void* v_new, void* k_pages, void* v_pages, int num_pages,
                             const int* block_table, int max_pages, int page_size,
                             const int* seq_lens, float k_scale, float v_scale, const void* gate,
                             const float* q_norm_w, const float* k_norm_w, void* out,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  zg::CacheMap map{};
  const int st = check_pages(num_pages, block_table, max_pages, page_size, map);
  if (st != ZG_OK) return st;
  return decode_impl(p, q, k_new, v_new, k_pages, v_pages, seq_lens, max_pages * page_size, 0,
                     map, gate, q_norm_w, k_norm_w, out, num_splits, workspace, workspace_bytes,
                     stream, 1, k_scale, v_scale);
}

int zg_attn_kv_write_pages(const zg_attn_params* p, const void* k_prime, const void* v,
                           void* k_pages, void* v_pages, int num_pages, const int* block_table,
                           int max_pages, int page_size, void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  zg::CacheMap map{};
  st = check_pages(num_pages, block_table, max_pages, page_size, map);
  if (st != ZG_OK) return st;
  if ((long long)p->seqlen > (long long)max_pages * page_size) return ZG_ERR_INVALID;
  if (p->batch == 0 || p->seqlen == 0) return ZG_OK;
  if (!k_prime || !v || !k_pages || !v_pages) return ZG_ERR_INVALID;
  if (!aligned16(k_prime) || !aligned16(v) || !aligned16(k_pages) || !aligned16(v_pages))
    return ZG_ERR_INVALID;
  return hip_status(zg::launch_kv_write_pages(
      static_cast<const uint16_t*>(k_prime), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(k_pages), static_cast<uint16_t*>(v_pages), p->batch, p->seqlen,
      p->n_kv_heads, map, reinterpret_cast<hipStream_t>(stream)));
}

int zg_linear(int M, int N, int K, const void* x, const void* w, void* y, void* stream) {
  if (M < 0 || N < 0 || K < 0) return ZG_ERR_INVALID;
  if (M == 0 || N == 0) return ZG_OK;
  if (N % 256 || K % 32 || K == 0) return ZG_ERR_UNSUPPORTED;
  if ((long long)K * 2 * 256 > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (!x || !w || !y) return ZG_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return ZG_ERR_INVALID;
  zg::GemmParams gp{};
  gp.a = static_cast<const uint16_t*>(x);
  gp.b = static_cast<const uint16_t*>(w);
  gp.M = M;
  gp.N = N;
  gp.K = K;
  gp.lda = K;
  gp.ldb = K;
  gp.seg[0] = zg::GemmSeg{static_cast<uint16_t*>(y), 0, N};
  gp.nseg = 1;
  return hip_status(zg::launch_gemm_bf16_tn(gp, reinterpret_cast<hipStream_t>(stream)));
}

int zg_quantize_fp8(long long n, const void* x, float scale, void* q, void* stream) {
  if (n < 0 || !(isfinite(scale) && scale > 0.f)) return ZG_ERR_INVALID;
  if (n == 0) return ZG_OK;
  if (n % 8) return ZG_ERR_UNSUPPORTED;
  if (!x || !q || !aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)) return ZG_ERR_INVALID;
  return hip_status(zg::launch_quantize_fp8(static_cast<const uint16_t*>(x),
                                            static_cast<uint8_t*>(q), n, scale,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int zg_linear_fp8(int M, int N, int K, const void* xq, const void* wq, float out_scale, void* y,
                  void* stream) {
  if (M < 0 || N < 0 || K < 0 || !isfinite(out_scale)) return ZG_ERR_INVALID;
  if (M == 0 || N == 0) return ZG_OK;
  if (N % 256 || K % 128 || K == 0) return ZG_ERR_UNSUPPORTED;
  if ((long long)K * 256 > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (!xq || !wq || !y) return ZG_ERR_INVALID;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y)) return ZG_ERR_INVALID;
  zg::GemmParams gp{};
  gp.a = static_cast<const uint16_t*>(xq);
  gp.b = static_cast<const uint16_t*>(wq);
  gp.M = M;
  gp.N = N;
  gp.K = K;
  gp.lda = K;
  gp.ldb = K;
  gp.seg[0] = zg::GemmSeg{static_cast<uint16_t*>(y), 0, N};
  gp.nseg = 1;
  gp.fp8 = 1;
  gp.out_scale = out_scale;
  return hip_status(zg::launch_gemm_bf16_tn(gp, reinterpret_cast<hipStream_t>(stream)));
}

int zg_qkvg_proj(const zg_attn_params* p, int hidden, const void* x, const void* w, void* q,
                 void* k, void* v, void* gate, void* stream) {
  int st = check_params(p);
  if (st != ZG_OK) return st;
  if (hidden < 0) return ZG_ERR_INVALID;
  const long long T = (long long)p->batch * p->seqlen;
  if (T == 0) return ZG_OK;
  if (T > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  const int nq = p->n_q_heads * kD, nk = p->n_kv_heads * kD;
  if (nk % 256 || hidden % 32 || hidden == 0) return ZG_ERR_UNSUPPORTED;
  if ((long long)hidden * 2 * 256 > 0x7fffffffLL) return ZG_ERR_UNSUPPORTED;
  if (!x || !w || !q || !k || !v) return ZG_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      (gate && !aligned16(gate)))
    return ZG_ERR_INVALID;
  zg::GemmParams gp{};
  gp.a = static_cast<const uint16_t*>(x);
  gp.b = static_cast<const uint16_t*>(w);
  gp.M = (int)T;
  gp.N = 2 * nk + (gate ? 2 * nq : nq);
  gp.K = hidden;
  gp.lda = hidden;
  gp.ldb = hidden;
  gp.seg[0] = zg::GemmSeg{static_cast<uint16_t*>(q), 0, nq};
  gp.seg[1] = zg::GemmSeg{static_cast<uint16_t*>(k), nq, nk};
  gp.seg[2] = zg::GemmSeg{static_cast<uint16_t*>(v), nq + nk, nk};
  gp.nseg = 3;
  if (gate) {
    gp.seg[3] = zg::GemmSeg{static_cast<uint16_t*>(gate), nq + 2 * nk, nq};
    gp.nseg = 4;
  }
  return hip_status(zg::launch_gemm_bf16_tn(gp, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
