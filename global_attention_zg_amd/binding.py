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
ZG_ERR_TOO_LARGE = -5


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


class DecodeLayer(ctypes.Structure):
    """One layer of a block decode step (zg_decode_layer)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k_new", "v_new", "k_cache", "v_cache",
                                                "gate", "q_norm_w", "k_norm_w", "out")] + \
               [("cache_cap", ctypes.c_int), ("ring", ctypes.c_int), ("window", ctypes.c_int)]


DECODE_BLOCK_MAX_LAYERS = 6


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
    lib.zg_attn_fwd_fp8_workspace_size.argtypes = [P]
    lib.zg_attn_fwd_fp8_workspace_size.restype = sz
    lib.zg_attn_fwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz,
                                    vp]
    lib.zg_attn_fwd_fp8.restype = i
    lib.zg_attn_decode_num_splits.argtypes = [P, i]
    lib.zg_attn_decode_num_splits.restype = i
    lib.zg_attn_decode_workspace_size.argtypes = [P, i, i]
    lib.zg_attn_decode_workspace_size.restype = sz
    lib.zg_attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, vp, i, vp, sz, vp]
    lib.zg_attn_decode.restype = i
    lib.zg_attn_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, vp, i, vp]
    lib.zg_attn_decode_noalloc.restype = i
    LP = ctypes.POINTER(DecodeLayer)
    lib.zg_attn_decode_block_num_splits.argtypes = [P, i]
    lib.zg_attn_decode_block_num_splits.restype = i
    lib.zg_attn_decode_block_workspace_size.argtypes = [P, i, LP]
    lib.zg_attn_decode_block_workspace_size.restype = sz
    lib.zg_attn_decode_block.argtypes = [P, i, LP, vp, vp, sz, vp]
    lib.zg_attn_decode_block.restype = i
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
            "zg_attn_decode_fp8", "zg_attn_decode_paged_fp8", "zg_attn_decode_noalloc",
            "zg_attn_fwd_fp8_workspace_size", "zg_attn_fwd_fp8",
            "zg_attn_decode_block_num_splits", "zg_attn_decode_block_workspace_size",
            "zg_attn_decode_block", "zg_attn_strerror")


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


class _Args:
    """Checks of a call's tensor arguments before their pointers go to the
    library: first each tensor's dtype, shape and layout as the C ABI
    documents them, then (done()) that every one is on the same CUDA device.
    Raises ValueError; None is accepted only where the C ABI takes NULL."""

    def __init__(self):
        self.seen = []

    def req(self, t, name, dtype, shape=None, optional=False):
        if t is None:
            if optional:
                return
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        dts = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in dts:
            raise ValueError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.seen.append((t, name))

    def done(self):
        dev = None
        for t, name in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name} must be on a CUDA device")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, expected {dev}")


BF16 = torch.bfloat16
F32 = torch.float32
I32 = torch.int32
U8 = torch.uint8


def _dims(t, name, n):
    if not isinstance(t, torch.Tensor) or t.dim() != n:
        raise ValueError(f"{name} must be a {n}-d tensor")
    return tuple(t.shape)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# The causal kernel's work-queue counters at the end of a global layer's
# forward workspace (also needed when K' goes to k_out).
QUEUE_BYTES = 256


def _fwd_workspace(full_bytes, k_out, causal, workspace, device):
    need = full_bytes if k_out is None else (QUEUE_BYTES if causal else 0)
    if workspace is None and need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ws_bytes


def zg_attn_fwd_workspace_size(p: Params) -> int:
    return int(_lib.zg_attn_fwd_workspace_size(ctypes.byref(p)))


def zg_attn_fwd(q, k, v, gate, q_norm_w, k_norm_w, *, window, rope_dim=42, rope_theta=10000.0,
                rms_eps=1e-6, softmax_scale=0.0, pos_offset=0, out=None, lse=None,
                want_lse=False, k_out=None, workspace=None, stream=None):
    """q [B,S,Hq,128], k/v [B,S,Hkv,128], gate [B,S,Hq,128] or None (bf16, CUDA);
    norm weights fp32 [128].  Returns (out, lse or None)."""
    B, S, Hq, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    a = _Args()
    a.req(q, "q", BF16)
    a.req(k, "k", BF16, (B, S, Hkv, D))
    a.req(v, "v", BF16, (B, S, Hkv, D))
    a.req(gate, "gate", BF16, (B, S, Hq, D), optional=True)
    a.req(q_norm_w, "q_norm_w", F32, (D,))
    a.req(k_norm_w, "k_norm_w", F32, (D,))
    a.req(out, "out", BF16, (B, S, Hq, D), optional=True)
    a.req(lse, "lse", F32, (B, Hq, S), optional=True)
    a.req(k_out, "k_out", BF16, (B, S, Hkv, D), optional=True)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
    p = make_params(B, S, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    workspace, ws_bytes = _fwd_workspace(zg_attn_fwd_workspace_size(p), k_out, window == 0,
                                         workspace, q.device)
    st = _lib.zg_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(q_norm_w),
                          _ptr(k_norm_w), _ptr(out), _ptr(lse), _ptr(k_out), _ptr(workspace),
                          ws_bytes, _stream(stream))
    _check(st)
    return out, lse


def zg_attn_fwd_fp8_workspace_size(p: Params) -> int:
    return int(_lib.zg_attn_fwd_fp8_workspace_size(ctypes.byref(p)))


def zg_attn_fwd_fp8(q, k, v, gate, q_norm_w, k_norm_w, *, k_scale, window=0, rope_dim=42,
                    rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0, pos_offset=0, out=None,
                    lse=None, want_lse=False, k_out=None, workspace=None, stream=None):
    """The E4M3 forward of a global layer: arguments as zg_attn_fwd, plus the
    per-tensor k_scale; k_out (optional) receives the uint8 K' codes
    [B,S,Hkv,128].  Returns (out, lse or None)."""
    B, S, Hq, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    a = _Args()
    a.req(q, "q", BF16)
    a.req(k, "k", BF16, (B, S, Hkv, D))
    a.req(v, "v", BF16, (B, S, Hkv, D))
    a.req(gate, "gate", BF16, (B, S, Hq, D), optional=True)
    a.req(q_norm_w, "q_norm_w", F32, (D,))
    a.req(k_norm_w, "k_norm_w", F32, (D,))
    a.req(out, "out", BF16, (B, S, Hq, D), optional=True)
    a.req(lse, "lse", F32, (B, Hq, S), optional=True)
    a.req(k_out, "k_out", U8, (B, S, Hkv, D), optional=True)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
    p = make_params(B, S, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    workspace, ws_bytes = _fwd_workspace(zg_attn_fwd_fp8_workspace_size(p), k_out, True,
                                         workspace, q.device)
    st = _lib.zg_attn_fwd_fp8(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                              _ptr(q_norm_w), _ptr(k_norm_w), float(k_scale), _ptr(out),
                              _ptr(lse), _ptr(k_out), _ptr(workspace), ws_bytes, _stream(stream))
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
    T, Hq, D = _dims(q, "q", 3)
    Hkv = _dims(k, "k", 3)[1]
    a = _Args()
    a.req(q, "q", BF16)
    a.req(k, "k", BF16, (T, Hkv, D))
    a.req(v, "v", BF16, (T, Hkv, D))
    a.req(gate, "gate", BF16, (T, Hq, D), optional=True)
    a.req(q_norm_w, "q_norm_w", F32, (D,))
    a.req(k_norm_w, "k_norm_w", F32, (D,))
    a.req(cu_seqlens, "cu_seqlens", I32, None)
    a.req(out, "out", BF16, (T, Hq, D), optional=True)
    a.req(lse, "lse", F32, (Hq, T), optional=True)
    a.req(k_out, "k_out", BF16, (T, Hkv, D), optional=True)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
    B = cu_seqlens.numel() - 1
    p = make_params(B, max_seqlen, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps,
                    softmax_scale, pos_offset)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    workspace, ws_bytes = _fwd_workspace(zg_attn_fwd_varlen_workspace_size(p, T), k_out,
                                         window == 0, workspace, q.device)
    st = _lib.zg_attn_fwd_varlen(ctypes.byref(p), _ptr(cu_seqlens), T, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out), _ptr(lse),
                                 _ptr(k_out), _ptr(workspace), ws_bytes, _stream(stream))
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
    B, S, Hq, D = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[2]
    a = _Args()
    a.req(q, "q", BF16)
    for t, n in ((k, "k"), (v, "v")):
        a.req(t, n, BF16, (B, S, Hkv, D))
    for t, n in ((out, "out"), (dout, "dout")):
        a.req(t, n, BF16, (B, S, Hq, D))
    a.req(gate, "gate", BF16, (B, S, Hq, D), optional=True)
    a.req(q_norm_w, "q_norm_w", F32, (D,))
    a.req(k_norm_w, "k_norm_w", F32, (D,))
    a.req(lse, "lse", F32, (B, Hq, S))
    a.req(dq, "dq", BF16, (B, S, Hq, D), optional=True)
    a.req(dk, "dk", BF16, (B, S, Hkv, D), optional=True)
    a.req(dv, "dv", BF16, (B, S, Hkv, D), optional=True)
    a.req(dgate, "dgate", BF16, (B, S, Hq, D), optional=True)
    a.req(dq_norm_w, "dq_norm_w", F32, (D,), optional=True)
    a.req(dk_norm_w, "dk_norm_w", F32, (D,), optional=True)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
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


def _check_decode(q, k_new, v_new, caches, seq_lens, gate, q_norm_w, k_norm_w, out, Hkv,
                  cache_dtype, block_table=None):
    B, Hq, D = _dims(q, "q", 3)
    a = _Args()
    a.req(q, "q", BF16)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        a.req(t, n, BF16, (B, Hkv, D), optional=True)
    shape = tuple(caches[0].shape) if isinstance(caches[0], torch.Tensor) else None
    for t, n in zip(caches, ("k_cache", "v_cache")):
        a.req(t, n, cache_dtype, shape)
    if shape is None or len(shape) != 4 or shape[1] != Hkv or shape[3] != D:
        raise ValueError(f"caches must be [*, {Hkv}, *, {D}]")
    if block_table is None and shape[0] != B:
        raise ValueError(f"caches must hold {B} sequences, got {shape[0]}")
    if block_table is not None:
        a.req(block_table, "block_table", I32, None)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be [{B}, max_pages]")
    a.req(seq_lens, "seq_lens", I32, (B,))
    a.req(gate, "gate", BF16, (B, Hq, D), optional=True)
    a.req(q_norm_w, "q_norm_w", F32, (D,))
    a.req(k_norm_w, "k_norm_w", F32, (D,))
    a.req(out, "out", BF16, (B, Hq, D), optional=True)
    return a


def zg_attn_decode_num_splits(p: Params, cache_cap: int) -> int:
    return int(_lib.zg_attn_decode_num_splits(ctypes.byref(p), cache_cap))


def zg_attn_decode_workspace_size(p: Params, cache_cap: int, num_splits: int = 0) -> int:
    return int(_lib.zg_attn_decode_workspace_size(ctypes.byref(p), cache_cap, num_splits))


def zg_attn_decode(q, k_new, v_new, k_cache, v_cache, seq_lens, *, ring, window, gate, q_norm_w,
                   k_norm_w, rope_dim=42, rope_theta=10000.0, rms_eps=1e-6, softmax_scale=0.0,
                   pos_offset=0, num_splits=0, out=None, workspace=None, stream=None):
    """q [B,Hq,128]; k_new/v_new [B,Hkv,128] or None; caches [B,Hkv,cap,128]
    (updated in place); seq_lens int32 [B] on the device.  Returns out."""
    _dims(k_cache, "k_cache", 4)
    a = _check_decode(q, k_new, v_new, (k_cache, v_cache), seq_lens, gate, q_norm_w, k_norm_w, out,
                  k_cache.shape[1], BF16)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
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


def _block_layers(layers, seq_lens):
    """Check every layer's tensors (as zg_attn_decode does, all layers with
    the same batch, heads and device) and build the zg_decode_layer array."""
    if not 1 <= len(layers) <= DECODE_BLOCK_MAX_LAYERS:
        raise ValueError(f"1 to {DECODE_BLOCK_MAX_LAYERS} layers")
    arr = (DecodeLayer * len(layers))()
    first = None
    a_all = _Args()
    for i, L in enumerate(layers):
        q, kc = L["q"], L["k_cache"]
        _dims(kc, f"layers[{i}].k_cache", 4)
        a = _check_decode(q, L.get("k_new"), L.get("v_new"), (kc, L["v_cache"]), seq_lens,
                          L.get("gate"), L["q_norm_w"], L["k_norm_w"], L.get("out"), kc.shape[1],
                          BF16)
        a.done()
        a_all.seen.extend(a.seen)
        dims = (q.shape[0], q.shape[1], kc.shape[1])
        if first is None:
            first = dims
        elif dims != first:
            raise ValueError(f"layers[{i}] has (B, Hq, Hkv) {dims}, layer 0 {first}")
        if L.get("out") is None:
            L["out"] = torch.empty_like(q)
        arr[i] = DecodeLayer(q.data_ptr(), None if L.get("k_new") is None else L["k_new"].data_ptr(),
                             None if L.get("v_new") is None else L["v_new"].data_ptr(),
                             kc.data_ptr(), L["v_cache"].data_ptr(),
                             None if L.get("gate") is None else L["gate"].data_ptr(),
                             L["q_norm_w"].data_ptr(), L["k_norm_w"].data_ptr(), L["out"].data_ptr(),
                             kc.shape[2], int(L["ring"]), int(L["window"]))
    a_all.done()
    return arr, first


def zg_attn_decode_block_num_splits(p: Params, cache_cap: int) -> int:
    return int(_lib.zg_attn_decode_block_num_splits(ctypes.byref(p), cache_cap))


def zg_attn_decode_block_workspace_size(p: Params, arr) -> int:
    return int(_lib.zg_attn_decode_block_workspace_size(ctypes.byref(p), len(arr), arr))


def zg_attn_decode_block(layers, seq_lens, *, rope_dim=42, rope_theta=10000.0, rms_eps=1e-6,
                         softmax_scale=0.0, pos_offset=0, workspace=None, stream=None):
    """One decode step of up to 6 layers in one launch.  layers: dicts with
    q, k_new, v_new (or None), k_cache, v_cache, gate (or None), q_norm_w,
    k_norm_w, ring, window and optionally out (else allocated and stored in
    the dict).  The workspace (uint8) must be zero-filled before its first
    step; a new one is.  Returns the list of outputs."""
    arr, (B, Hq, Hkv) = _block_layers(layers, seq_lens)
    p = make_params(B, 0, Hq, Hkv, 128, 0, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    nbytes = zg_attn_decode_block_workspace_size(p, arr)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=layers[0]["q"].device)
    else:
        a = _Args()
        a.req(workspace, "workspace", U8, None)
        a.done()
    st = _lib.zg_attn_decode_block(ctypes.byref(p), len(arr), arr, _ptr(seq_lens), _ptr(workspace),
                                   workspace.numel(), _stream(stream))
    _check(st)
    return [L["out"] for L in layers]


def zg_attn_decode_noalloc(q, k_new, v_new, k_cache, v_cache, seq_lens, *, ring, window, gate,
                           q_norm_w, k_norm_w, rope_dim=42, rope_theta=10000.0, rms_eps=1e-6,
                           softmax_scale=0.0, pos_offset=0, num_splits=0, out=None, stream=None):
    """zg_attn_decode with the split partials in the library's static scratch
    (no workspace).  Returns out."""
    _dims(k_cache, "k_cache", 4)
    a = _check_decode(q, k_new, v_new, (k_cache, v_cache), seq_lens, gate, q_norm_w, k_norm_w, out,
                  k_cache.shape[1], BF16)
    a.done()
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, 0, Hq, Hkv, D, window, rope_dim, rope_theta, rms_eps, softmax_scale,
                    pos_offset)
    if out is None:
        out = torch.empty_like(q)
    st = _lib.zg_attn_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), cap, int(ring),
                                     _ptr(gate), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(out),
                                     num_splits, _stream(stream))
    _check(st)
    return out


def zg_attn_kv_write_pages(k_prime, v, k_pages, v_pages, block_table, *, stream=None):
    """k_prime / v [B,S,Hkv,128] (K' from zg_attn_fwd's k_out, and V) into the
    page pool k_pages / v_pages [num_pages,Hkv,page_size,128]; block_table
    int32 [B,max_pages] on the device."""
    B, S, Hkv, D = _dims(k_prime, "k_prime", 4)
    a = _Args()
    a.req(k_prime, "k_prime", BF16)
    a.req(v, "v", BF16, (B, S, Hkv, D))
    np_, _, ps, _ = _dims(k_pages, "k_pages", 4)
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        a.req(t, n, BF16, (np_, Hkv, ps, D))
    a.req(block_table, "block_table", I32, None)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [{B}, max_pages]")
    a.done()
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
    _dims(k_pages, "k_pages", 4)
    a = _check_decode(q, k_new, v_new, (k_pages, v_pages), seq_lens, gate, q_norm_w, k_norm_w, out,
                  k_pages.shape[1], BF16, block_table)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
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
    _dims(k_cache, "k_cache", 4)
    a = _check_decode(q, k_new, v_new, (k_cache, v_cache), seq_lens, gate, q_norm_w, k_norm_w, out,
                  k_cache.shape[1], U8)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
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
    _dims(k_pages, "k_pages", 4)
    a = _check_decode(q, k_new, v_new, (k_pages, v_pages), seq_lens, gate, q_norm_w, k_norm_w, out,
                  k_pages.shape[1], U8, block_table)
    a.req(workspace, "workspace", U8, None, optional=True)
    a.done()
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
    M, K = _dims(x, "x", 2)
    a = _Args()
    a.req(x, "x", BF16)
    a.req(w, "w", BF16, (_dims(w, "w", 2)[0], K))
    a.req(out, "out", BF16, (M, w.shape[0]), optional=True)
    a.done()
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(_lib.zg_linear(M, N, K, _ptr(x), _ptr(w), _ptr(out), _stream(stream)))
    return out


def zg_qkvg_proj(x, w, n_q_heads, n_kv_heads, gated, *, q=None, k=None, v=None, gate=None,
                 stream=None):
    """x [T,hidden] bf16, w [Nw,hidden] stacking W_q, W_k, W_v (and W_g when
    gated).  Returns (q [T,Hq,128], k [T,Hkv,128], v, gate or None)."""
    T, hidden = _dims(x, "x", 2)
    a = _Args()
    a.req(x, "x", BF16)
    nw = (n_q_heads * (2 if gated else 1) + 2 * n_kv_heads) * 128
    a.req(w, "w", BF16, (nw, hidden))
    for t, n, h in ((q, "q", n_q_heads), (k, "k", n_kv_heads), (v, "v", n_kv_heads),
                    (gate, "gate", n_q_heads)):
        a.req(t, n, BF16, (T, h, 128), optional=True)
    a.done()
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
    a = _Args()
    a.req(x, "x", BF16)
    a.req(out, "out", U8, tuple(x.shape), optional=True)
    a.done()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.zg_quantize_fp8(x.numel(), _ptr(x), float(scale), _ptr(out), _stream(stream)))
    return out


def zg_linear_fp8(xq, wq, out_scale, out=None, stream=None):
    """E4M3 codes xq [M,K], wq [N,K] (uint8) -> y [M,N] bf16 = out_scale * xq . wq^T."""
    M, K = _dims(xq, "xq", 2)
    a = _Args()
    a.req(xq, "xq", U8)
    a.req(wq, "wq", U8, (_dims(wq, "wq", 2)[0], K))
    a.req(out, "out", BF16, (M, wq.shape[0]), optional=True)
    a.done()
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(_lib.zg_linear_fp8(M, N, K, _ptr(xq), _ptr(wq), float(out_scale), _ptr(out),
                              _stream(stream)))
    return out
