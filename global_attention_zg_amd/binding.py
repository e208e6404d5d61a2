"""Thin ctypes binding over libzgattn.so (C ABI in include/zg_attn.h).

Argument marshalling only: tensors are passed as device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  torch is used for device memory (outputs, workspace) and streams.
Importing this module loads the library and raises if it is missing: there is
no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzgattn.so")

ZG_OK = 0
ZG_ERR_INVALID = -1
ZG_ERR_UNSUPPORTED = -2
ZG_ERR_WORKSPACE = -3
ZG_ERR_HIP = -4


class ZgAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"zg_attn status {status}: {msg}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int),
        ("seqlen", ctypes.c_int),
        ("n_q_heads", ctypes.c_int),
        ("n_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("window", ctypes.c_int),
        ("rope_dim", ctypes.c_int),
        ("rope_theta", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("pos_offset", ctypes.c_longlong),
    ]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run global_attention_zg_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.zg_attn_fwd_workspace_size.argtypes = [P]
    lib.zg_attn_fwd_workspace_size.restype = sz
    lib.zg_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.zg_attn_fwd.restype = i
    ll = ctypes.c_longlong
    lib.zg_attn_fwd_varlen_workspace_size.argtypes = [P, ll]
    lib.zg_attn_fwd_varlen_workspace_size.restype = sz
    lib.zg_attn_fwd_varlen.argtypes = [P, vp, ll, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.zg_attn_fwd_varlen.restype = i
    lib.zg_attn_decode_num_splits.argtypes = [P, i]
    lib.zg_attn_decode_num_splits.restype = i
    lib.zg_attn_decode_workspace_size.argtypes = [P, i, i]
    lib.zg_attn_decode_workspace_size.restype = sz
    lib.zg_attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, vp, i, vp, sz, vp]
    lib.zg_attn_decode.restype = i
    lib.zg_attn_decode_paged.argtypes = [P, vp, vp, vp, vp, vp, i, vp, i, i, vp, vp, vp, vp, vp,
                                         i, vp, sz, vp]
    lib.zg_attn_decode_paged.restype = i
    f = ctypes.c_float
    lib.zg_attn_decode_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, i, i, f, f, vp, vp, vp, vp, i,
                                       vp, sz, vp]
    lib.zg_attn_decode_fp8.restype = i
    lib.zg_attn_decode_paged_fp8.argtypes = [P, vp, vp, vp, vp, vp, i, vp, i, i, vp, f, f, vp, vp,
                                             vp, vp, i, vp, sz, vp]
    lib.zg_attn_decode_paged_fp8.restype = i
    lib.zg_attn_kv_write_pages.argtypes = [P, vp, vp, vp, vp, i, vp, i, i, vp]
    lib.zg_attn_kv_write_pages.restype = i
    lib.zg_linear.argtypes = [i, i, i, vp, vp, vp, vp]
    lib.zg_linear.restype = i
    lib.zg_qkvg_proj.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp]
    lib.zg_qkvg_proj.restype = i
    lib.zg_quantize_fp8.argtypes = [ctypes.c_longlong, vp, ctypes.c_float, vp, vp]
    lib.zg_quantize_fp8.restype = i
    lib.zg_linear_fp8.argtypes = [i, i, i, vp, vp, ctypes.c_float, vp, vp]
    lib.zg_linear_fp8.restype = i
    lib.zg_attn_bwd_workspace_size.argtypes = [P]
    lib.zg_attn_bwd_workspace_size.restype = sz
    lib.zg_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                sz, vp]
    lib.zg_attn_bwd.restype = i
    lib.zg_attn_strerror.argtypes = [i]
    lib.zg_attn_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()

EXPORTED = ("zg_attn_fwd_workspace_size", "zg_attn_fwd", "zg_attn_fwd_varlen_workspace_size",
            "zg_attn_fwd_varlen", "zg_attn_decode_num_splits",
            "zg_attn_decode_workspace_size", "zg_attn_decode", "zg_attn_kv_write_pages",
            "zg_attn_decode_paged", "zg_attn_bwd_workspace_size", "zg_attn_bwd",
            "zg_linear", "zg_qkvg_proj", "zg_quantize_fp8", "zg_linear_fp8",
            "zg_attn_decode_fp8", "zg_attn_decode_paged_fp8", "zg_attn_strerror")


def library_path() -> str:
    return _LIB_PATH


def zg_attn_strerror(status: int) -> str:
    return _lib.zg_attn_strerror(status).decode()


def _check(status: int):
    if status != ZG_OK:
        raise ZgAttnError(status, zg_attn_strerror(status))


def make_params(batch, seqlen, n_q_heads, n_kv_heads, head_dim=128, window=0, rope_dim=42,
                rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0, pos_offset=0) -> Params:
    return Params(batch, seqlen, n_q_heads, n_kv_heads, head_dim, window, rope_dim,
                  rope_theta, rms_eps, softmax_scale, pos_offset)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def zg_attn_fwd_workspace_size(p: Params) -> int:
    return int(_lib.zg_attn_fwd_workspace_size(ctypes.byref(p)))


def zg_attn_fwd(q, k, v, gate, q_norm_w, k_norm_w, *, window, rope_dim=42, rope_theta=10000.0,
                rms_eps=1e-6, softmax_scale=0.0, pos_offset=0, out=None, lse=None,
                want_lse=False, k_out=None, workspace=None, stream=None):
    """q [B,S,Hq,128], k/v [B,S,Hkv,128], gate [B,S,Hq,128] or None (bf16, CUDA);
    norm weights fp32 [128].  Returns (out, lse or None)."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    p = make_params(B, S, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    ws_bytes = 0
    if k_out is None:
        ws_bytes = zg_attn_fwd_workspace_size(p)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w),
                          _ptr(k_norm_w), _ptr(out), _ptr(lse), _ptr(k_out),
                          _ptr(workspace) if k_out is None else None, ws_bytes, _stream(stream))
    _check(st)
    return out, lse


def zg_attn_fwd_varlen_workspace_size(p: Params, total_tokens: int) -> int:
    return int(_lib.zg_attn_fwd_varlen_workspace_size(ctypes.byref(p), total_tokens))


def zg_attn_fwd_varlen(q, k, v, gate, q_norm_w, k_norm_w, cu_seqlens, max_seqlen, *, window,
                       rope_dim=42, rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0,
                       pos_offset=0, out=None, lse=None, want_lse=False, k_out=None,
                       workspace=None, stream=None):
    """Packed batch: q [T,Hq,128], k/v [T,Hkv,128], gate [T,Hq,128] or None;
    cu_seqlens int32 [B+1] on the device.  Returns (out, lse [Hq,T] or None)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = cu_seqlens.numel() - 1
    p = make_params(B, max_seqlen, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps,
                    softmax_scale, pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    ws_bytes = 0
    if k_out is None:
        ws_bytes = zg_attn_fwd_varlen_workspace_size(p, T)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_fwd_varlen(ctypes.byref(p), _ptr(cu_seqlens), T, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), _ptr(lse),
                                 _ptr(k_out), _ptr(workspace) if k_out is None else None,
                                 ws_bytes, _stream(stream))
    _check(st)
    return out, lse


def zg_attn_bwd_workspace_size(p: Params) -> int:
    return int(_lib.zg_attn_bwd_workspace_size(ctypes.byref(p)))


def zg_attn_bwd(q, k, v, gate, q_norm_w, k_norm_w, out, lse, dout, *, window, rope_dim=42,
                rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0, pos_offset=0, dq=None,
                dk=None, dv=None, dgate=None, dq_norm_w=None, dk_norm_w=None, workspace=None,
                stream=None):
    """Gradients of sum(dout * out) for out, lse = zg_attn_fwd(...) with the same
    inputs.  Returns a dict: dq, dk, dv, dgate (None when gate is None),
    dq_norm_w, dk_norm_w."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    p = make_params(B, S, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if gate is not None and dgate is None:
        dgate = torch.empty_like(gate)
    if dq_norm_w is None:
        dq_norm_w = torch.empty(D, dtype=torch.float32, device=q.device)
    if dk_norm_w is None:
        dk_norm_w = torch.empty(D, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = zg_attn_bwd_workspace_size(p)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w),
                          _ptr(k_norm_w), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(dgate), _ptr(dq_norm_w), _ptr(dk_norm_w),
                          _ptr(workspace), ws_bytes, _stream(stream))
    _check(st)
    return {"dq": dq, "dk": dk, "dv": dv, "dgate": dgate if gate is not None else None,
            "dq_norm_w": dq_norm_w, "dk_norm_w": dk_norm_w}


def zg_attn_decode_num_splits(p: Params, cache_cap: int) -> int:
    return int(_lib.zg_attn_decode_num_splits(ctypes.byref(p), cache_cap))


def zg_attn_decode_workspace_size(p: Params, cache_cap: int, num_splits: int = 0) -> int:
    return int(_lib.zg_attn_decode_workspace_size(ctypes.byref(p), cache_cap, num_splits))


def zg_attn_decode(q, k_new, v_new, k_cache, v_cache, seq_lens, *, ring, window, gate, q_norm_w,
                   k_norm_w, rope_dim=42, rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0,
                   pos_offset=0, num_splits=0, out=None, workspace=None, stream=None):
    """q [B,Hq,128]; k_new/v_new [B,Hkv,128] or None; caches [B,Hkv,cap,128]
    (updated in place); seq_lens int32 [B] on the device.  Returns out."""
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, 0, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = zg_attn_decode_workspace_size(p, cap, num_splits)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_decode(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                             _ptr(v_cache), _ptr(seq_lens), cap, int(ring), _ptr(gate),
                             _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), num_splits,
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st)
    return out


def zg_attn_kv_write_pages(k_prime, v, k_pages, v_pages, block_table, *, stream=None):
    """k_prime / v [B,S,Hkv,128] (K' from zg_attn_fwd's k_out, and V) into the
    page pool k_pages / v_pages [num_pages,Hkv,page_size,128]; block_table
    int32 [B,max_pages] on the device."""
    B, S, Hkv, D = k_prime.shape
    num_pages, _, page_size, _ = k_pages.shape
    p = make_params(B, S, Hkv, Hkv, D)
    st = _lib.zg_attn_kv_write_pages(ctypes.byref(p), _ptr(k_prime), _ptr(v), _ptr(k_pages),
                                     _ptr(v_pages), num_pages, _ptr(block_table),
                                     block_table.shape[1], page_size, _stream(stream))
    _check(st)


def zg_attn_decode_paged(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, *, window,
                         gate, q_norm_w, k_norm_w, rope_dim=42, rope_theta=10000.0, rms_eps=1e-6,
                         softmax_scale=0.0, pos_offset=0, num_splits=0, out=None,
                         workspace=None, stream=None):
    """zg_attn_decode over a page pool [num_pages,Hkv,page_size,128] with an
    int32 block table [B,max_pages].  Returns out."""
    B, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    cap = max_pages * page_size
    p = make_params(B, 0, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = zg_attn_decode_workspace_size(p, cap, num_splits)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_pages), _ptr(v_pages), num_pages, _ptr(block_table),
                                   max_pages, page_size, _ptr(seq_lens), _ptr(gate),
                                   _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), num_splits,
                                   _ptr(workspace), ws_bytes, _stream(stream))
    _check(st)
    return out


def zg_attn_decode_fp8(q, k_new, v_new, k_cache, v_cache, seq_lens, *, ring, window, k_scale,
                       v_scale, gate, q_norm_w, k_norm_w, rope_dim=42, rope_theta=10000.0,
                       rms_eps=1e-6, softmax_scale=0.0, pos_offset=0, num_splits=0, out=None,
                       workspace=None, stream=None):
    """zg_attn_decode over an E4M3 cache: k_cache / v_cache uint8 [B,Hkv,cap,128]
    hold the codes of K' * k_scale and V * v_scale (updated in place).
    Returns out (bf16 [B,Hq,128])."""
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, 0, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = zg_attn_decode_workspace_size(p, cap, num_splits)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_decode_fp8(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new),
                                 _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), cap, int(ring),
                                 float(k_scale), float(v_scale), _ptr(gate), _ptr(q_norm_w),
                                 _ptr(k_norm_w), _ptr(out), num_splits, _ptr(workspace),
                                 ws_bytes, _stream(stream))
    _check(st)
    return out


def zg_attn_decode_paged_fp8(q, k_new, v_new, k_pages, v_pages, block_table, seq_lens, *,
                             window, k_scale, v_scale, gate, q_norm_w, k_norm_w, rope_dim=42,
                             rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0, pos_offset=0,
                             num_splits=0, out=None, workspace=None, stream=None):
    """zg_attn_decode_paged over E4M3 pages uint8 [num_pages,Hkv,page_size,128].
    Returns out."""
    B, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    cap = max_pages * page_size
    p = make_params(B, 0, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = zg_attn_decode_workspace_size(p, cap, num_splits)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.zg_attn_decode_paged_fp8(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new),
                                       _ptr(k_pages), _ptr(v_pages), num_pages,
                                       _ptr(block_table), max_pages, page_size, _ptr(seq_lens),
                                       float(k_scale), float(v_scale), _ptr(gate),
                                       _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), num_splits,
                                       _ptr(workspace), ws_bytes, _stream(stream))
    _check(st)
    return out


def zg_linear(x, w, out=None, stream=None):
    """y = x w^T: x [M,K], w [N,K] bf16 on the device -> y [M,N] bf16."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(_lib.zg_linear(M, N, K, _ptr(x), _ptr(w), _ptr(out), _stream(stream)))
    return out


def zg_qkvg_proj(x, w, n_q_heads, n_kv_heads, gated, *, q=None, k=None, v=None, gate=None,
                 stream=None):
    """x [T,hidden] bf16, w [Nw,hidden] stacking W_q, W_k, W_v (and W_g when
    gated).  Returns (q [T,Hq,128], k [T,Hkv,128], v, gate or None)."""
    T, hidden = x.shape
    D = 128
    p = make_params(1, T, n_q_heads, n_kv_heads, D)
    dev = x.device
    q = torch.empty((T, n_q_heads, D), dtype=x.dtype, device=dev) if q is None else q
    k = torch.empty((T, n_kv_heads, D), dtype=x.dtype, device=dev) if k is None else k
    v = torch.empty((T, n_kv_heads, D), dtype=x.dtype, device=dev) if v is None else v
    if gated and gate is None:
        gate = torch.empty((T, n_q_heads, D), dtype=x.dtype, device=dev)
    _check(_lib.zg_qkvg_proj(ctypes.byref(p), hidden, _ptr(x), _ptr(w), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(gate if gated else None), _stream(stream)))
    return q, k, v, (gate if gated else None)


def zg_quantize_fp8(x, scale, out=None, stream=None):
    """bf16 tensor -> uint8 tensor of E4M3 codes of x * scale (same shape)."""
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.zg_quantize_fp8(x.numel(), _ptr(x), float(scale), _ptr(out), _stream(stream)))
    return out


def zg_linear_fp8(xq, wq, out_scale, out=None, stream=None):
    """E4M3 codes xq [M,K], wq [N,K] (uint8) -> y [M,N] bf16 = out_scale * xq . wq^T."""
    M, K = xq.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(_lib.zg_linear_fp8(M, N, K, _ptr(xq), _ptr(wq), float(out_scale), _ptr(out),
                              _stream(stream)))
    return out
