"""Plain fp64 CPU oracle for the ZGCM-1 hybrid attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or falls back to it,
and this module imports nothing from the product package.

Sources, cited by page title and section:

* [RB] "ZGCM-1:面向数学与智能体搜索的全开源高效基础模型"
  (paper.rainbus.top/paper/2609.13356): section 前置知识 › 滑动窗口注意力(SWA)与
  混合注意力 (every token attends to its 128 neighbouring tokens; 27 gated SWA
  layers + 5 global layers at layers 6/12/18/24/30); section 核心方法 (GQA
  32 query / 8 KV heads, partial RoPE ratio 0.33, hidden 4096); the
  structured-data table, row "256K 上下文推理 KV 缓存" (5.0 GiB vs 32.0 GiB, 6.4x).
* [SB] "7B 打 235B？中关村学院把'小模型怎么活'这道题答成了一份全开源配方"
  (shibing624.github.io ai-paper-analysis): section 🏗️ 架构 (QK RMSNorm, GQA,
  RoPE ratio 0.33, 128-token gated SWA, sigmoid gate on the local output,
  KV 128 KiB -> 20 KiB per token); section 📊 数据与课程 (RoPE base 10M at 256K).

The pages give the method in prose only; the formula of the gate was lost when
the page was extracted.  Where the pages are silent this module takes the
plainest reading and says so in each function's docstring.

Everything is computed in float64 from the exact (bf16-representable) input
values.  Row blocking below is for memory only and changes no arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "linear",
    "qkvg_proj",
    "E4M3_MAX",
    "e4m3_decode",
    "quantize_e4m3",
    "e4m3_row_scale",
    "e4m3_rows",
    "attention_decode_fp8",
    "attention_fwd_fp8",
    "rms_norm",
    "rope_angles",
    "apply_partial_rope",
    "visible",
    "attention_fwd",
    "decode_group",
    "attention_decode",
    "rope_bwd",
    "rms_norm_bwd",
    "attention_bwd",
    "kv_cache_bytes_per_token",
    "kv_cache_bytes",
    "layer_schedule",
    "inband_pairs",
]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to float64 exactly."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Step 1: QK-RMSNorm  ([SB] 🏗️ 架构: queries and keys are RMS-normalised)
# ---------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (one attention head of D values).

    Reading: per-head statistics over the D = 128 dims, one weight vector of
    length D shared by all heads, multiplicative weight, epsilon added to the
    mean square:  x_hat = x / sqrt(mean(x^2) + eps) * gamma.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 2: partial RoPE  ([RB] 核心方法 / [SB] 🏗️ 架构: rotary ratio 0.33)
# ---------------------------------------------------------------------------
def rope_angles(positions: np.ndarray, rope_dim: int, theta: float) -> np.ndarray:
    """Rotation angles phi[p, j] = p * theta^(-2j/R) for j < R/2 (float64).

    Reading: the frequency exponent is taken over the R rotary dims, not over
    the whole head.
    """
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * j / float(rope_dim))
    return np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]


def apply_partial_rope(x: np.ndarray, positions: np.ndarray, rope_dim: int,
                       theta: float) -> np.ndarray:
    """Rotate the first ``rope_dim`` dims of every head; the rest pass through.

    ``x`` has shape [S, H, D] and ``positions`` shape [S].  Reading: the
    rotary dims are the first R = floor(0.33 * D) dims, paired rotate-half
    style as (j, j + R/2):
        y_j       = x_j cos(phi_j) - x_{j+R/2} sin(phi_j)
        y_{j+R/2} = x_{j+R/2} cos(phi_j) + x_j sin(phi_j)
    """
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    if rope_dim == 0:
        return y
    half = rope_dim // 2
    phi = rope_angles(positions, rope_dim, theta)  # [S, half]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:rope_dim]
    y[..., :half] = x1 * c - x2 * s
    y[..., half:rope_dim] = x2 * c + x1 * s
    return y


# ---------------------------------------------------------------------------
# Steps 3-7: banded / global causal GQA attention with the sigmoid gate
# ---------------------------------------------------------------------------
def visible(i: np.ndarray, j: np.ndarray, window: int) -> np.ndarray:
    """Key j is visible to query i iff j <= i and (window == 0 or i - j < window).

    Reading of [RB] 前置知识 (each token sees its 128 neighbouring tokens):
    the band holds 128 keys including the query itself; window == 0 means
    global causal attention.
    """
    ok = j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def _sigmoid(g: np.ndarray) -> np.ndarray:
    # 1 / (1 + e^-g): exact 1 at +inf and exact 0 at -inf.
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def attention_fwd(q, k, v, gate, q_norm_w, k_norm_w, *, window: int,
                  rope_dim: int, rope_theta: float, rms_eps: float,
                  softmax_scale: float = 0.0, pos_offset: int = 0,
                  rows=None, chunk: int = 1024, q_map=None, k_map=None):
    """Prefill / training forward of one attention layer, in float64.

    Shapes: q [B,S,Hq,D], k and v [B,S,Hkv,D], gate [B,S,Hq,D] or None,
    norm weights [D].  Returns (out [B,R,Hq,D], lse [B,Hq,R]) where R is S, or
    len(rows) when ``rows`` (sorted query indices) selects a sample.

    Per query head h the key/value head is h // (Hq // Hkv) (reading: GQA
    with contiguous groups).  Scores are tau * q'_i . k'_j with
    tau = softmax_scale or 1/sqrt(D) (reading), softmax over visible keys,
    out_i = sum_j P_ij v_j, then on a gated layer out_i *= sigmoid(G_i)
    elementwise (reading of the gate whose formula the page lost: the local
    attention output is multiplied by a sigmoid gate of the output's shape).
    LSE is the natural-log log-sum-exp of the scaled scores.

    ``q_map`` / ``k_map``, when given, are applied to the normalised, rotated
    query rows [r,Hq,D] / key rows [keys,Hkv,D] before the scores (the E4M3
    variant quantizes them there).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    tau = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    nr = len(rows)
    out = np.zeros((B, nr, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, nr), dtype=np.float64)
    pos = pos_offset + np.arange(S, dtype=np.int64)
    for b in range(B):
        # Keys needed: everything up to the last requested row.
        kmax = int(rows.max()) + 1 if nr else 0
        kn = rms_norm(k[b, :kmax], k_norm_w, rms_eps)
        kn = apply_partial_rope(kn, pos[:kmax], rope_dim, rope_theta)
        if k_map is not None:
            kn = k_map(kn)
        vb = v[b, :kmax]
        for c0 in range(0, nr, chunk):
            ridx = rows[c0:c0 + chunk]
            qn = rms_norm(q[b, ridx], q_norm_w, rms_eps)
            qn = apply_partial_rope(qn, pos[ridx], rope_dim, rope_theta)
            if q_map is not None:
                qn = q_map(qn)
            lo = 0 if window == 0 else max(0, int(ridx.min()) - window + 1)
            hi = int(ridx.max()) + 1
            jj = np.arange(lo, hi)
            mask = visible(ridx[:, None], jj[None, :], window)  # [r, keys]
            for g in range(Hkv):
                kg = kn[lo:hi, g, :]                  # [keys, D]
                vg = vb[lo:hi, g, :]
                for hh in range(grp):
                    h = g * grp + hh
                    s = tau * (qn[:, h, :] @ kg.T)    # [r, keys]
                    s = np.where(mask, s, -np.inf)
                    m = np.max(s, axis=1, keepdims=True)
                    e = np.exp(s - m)
                    den = np.sum(e, axis=1, keepdims=True)
                    o = (e @ vg) / den
                    if gate is not None:
                        o = o * _sigmoid(np.asarray(gate[b, ridx, h, :], dtype=np.float64))
                    out[b, c0:c0 + len(ridx), h, :] = o
                    lse[b, h, c0:c0 + len(ridx)] = (m + np.log(den))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# Step 8: decode = the last row of the forward over the cached keys
# ---------------------------------------------------------------------------
def decode_group(q_group, k_new, v_new, k_cache, v_cache, seq_len: int, *,
                 ring: bool, window: int, gate_group, q_norm_w, k_norm_w,
                 rope_dim: int, rope_theta: float, rms_eps: float,
                 softmax_scale: float = 0.0, pos_offset: int = 0, q_map=None):
    """One decode step for the query heads of ONE KV head of ONE sequence.

    q_group [G,D] raw new-token queries; k_new, v_new [D] raw new key/value
    or None when the new token is already in the cache; k_cache, v_cache
    [cap,D] cache contents before the append, K stored post-norm/RoPE.
    The new token sits at position p = pos_offset + seq_len - 1 and in cache
    slot seq_len-1 (linear cache) or (seq_len-1) % cap (ring).  Visible keys
    are the positions max(0, L-W)..L-1 (W = cap for a ring, W = window > 0
    for a banded linear cache, all of 0..L-1 for a global one).

    Returns (out [G,D], lse [G], k_appended [D] or None).  Reading: the
    cache holds K' (normalised and rotated at its own position) and decode is
    exactly row L-1 of ``attention_fwd`` over the same keys.  ``q_map``, when
    given, is applied to the normalised, rotated queries [G,D] before the
    scores (the E4M3 variant quantizes them there).
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    G, D = q_group.shape
    cap = k_cache.shape[0]
    L = int(seq_len)
    p = pos_offset + L - 1
    tau = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(D)
    W = cap if ring else window
    first = max(0, L - W) if W > 0 else 0
    positions = np.arange(first, L)
    slots = positions % cap if ring else positions
    kk = np.asarray(k_cache, dtype=np.float64)[slots].copy()
    vv = np.asarray(v_cache, dtype=np.float64)[slots].copy()
    k_app = None
    if k_new is not None:
        kn = rms_norm(np.asarray(k_new, dtype=np.float64)[None, None, :], k_norm_w, rms_eps)
        kn = apply_partial_rope(kn, np.array([p]), rope_dim, rope_theta)[0, 0]
        k_app = kn
        kk[-1] = kn
        vv[-1] = np.asarray(v_new, dtype=np.float64)
    qn = rms_norm(q_group[None], q_norm_w, rms_eps)
    qn = apply_partial_rope(qn, np.array([p]), rope_dim, rope_theta)[0]  # [G,D]
    if q_map is not None:
        qn = q_map(qn)
    s = tau * (qn @ kk.T)                       # [G, keys]
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    den = np.sum(e, axis=1, keepdims=True)
    o = (e @ vv) / den
    if gate_group is not None:
        o = o * _sigmoid(np.asarray(gate_group, dtype=np.float64))
    return o, (m + np.log(den))[:, 0], k_app


def attention_decode(q, k_new, v_new, k_cache, v_cache, seq_lens, *, ring: bool,
                     window: int, gate, q_norm_w, k_norm_w, rope_dim: int,
                     rope_theta: float, rms_eps: float, softmax_scale: float = 0.0,
                     pos_offset: int = 0):
    """Batched decode: q [B,Hq,D]; k_new, v_new [B,Hkv,D] or None;
    caches [B,Hkv,cap,D]; seq_lens [B]; gate [B,Hq,D] or None.

    Returns (out [B,Hq,D], lse [B,Hq], cache_k_after [B,Hkv,cap,D]) where the
    last is the K cache with the appended rows written in.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    k_after = np.array(k_cache, dtype=np.float64, copy=True)
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(Hkv):
            hs = slice(g * grp, (g + 1) * grp)
            o, ls, ka = decode_group(
                q[b, hs], None if k_new is None else k_new[b, g],
                None if v_new is None else v_new[b, g], k_cache[b, g], v_cache[b, g], L,
                ring=ring, window=window, gate_group=None if gate is None else gate[b, hs],
                q_norm_w=q_norm_w, k_norm_w=k_norm_w, rope_dim=rope_dim,
                rope_theta=rope_theta, rms_eps=rms_eps, softmax_scale=softmax_scale,
                pos_offset=pos_offset)
            out[b, hs] = o
            lse[b, hs] = ls
            if ka is not None:
                slot = (L - 1) % cap if ring else L - 1
                k_after[b, g, slot] = ka
    return out, lse, k_after


# ---------------------------------------------------------------------------
# Training backward: the derivative of steps 1-7.
#
# The pages measure the model in training ([RB] 前置知识 and the throughput
# ablation of the architecture section; [SB] 🏗️ 架构), but define only the
# forward computation.  The functions below are that forward's derivative by
# the chain rule, written out step by step; nothing in them is taken from
# the pages beyond the forward definitions above.
# ---------------------------------------------------------------------------
def rope_bwd(dy: np.ndarray, positions: np.ndarray, rope_dim: int,
             theta: float) -> np.ndarray:
    """Gradient through apply_partial_rope: each rotary pair (j, j+R/2) was
    rotated by phi_j, so its gradient is rotated back by -phi_j (the
    rotation is orthogonal); the other dims pass through."""
    dy = np.asarray(dy, dtype=np.float64)
    dx = dy.copy()
    if rope_dim == 0:
        return dx
    half = rope_dim // 2
    phi = rope_angles(positions, rope_dim, theta)
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    d1 = dy[..., :half]
    d2 = dy[..., half:rope_dim]
    dx[..., :half] = d1 * c + d2 * s
    dx[..., half:rope_dim] = d2 * c - d1 * s
    return dx


def rms_norm_bwd(x: np.ndarray, gamma: np.ndarray, eps: float, dxhat: np.ndarray):
    """Gradient through rms_norm over the last axis.

    With r = (mean(x^2) + eps)^(-1/2) and x_hat = x r gamma:
        dx     = r (gamma * dx_hat) - x r^3 mean(gamma * dx_hat * x)
        dgamma = sum over rows of dx_hat * x * r
    Returns (dx, dgamma).
    """
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    dxhat = np.asarray(dxhat, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gd = dxhat * gamma
    dx = r * gd - x * r ** 3 * np.mean(gd * x, axis=-1, keepdims=True)
    dgamma = np.sum((dxhat * x * r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dgamma


def attention_bwd(q, k, v, gate, q_norm_w, k_norm_w, dout, *, window: int,
                  rope_dim: int, rope_theta: float, rms_eps: float,
                  softmax_scale: float = 0.0, pos_offset: int = 0, chunk: int = 1024,
                  rows=None, keys=None):
    """Gradients of L = sum(dout * Y) for the layer Y = attention_fwd(...)[0].

    Returns a dict with dq, dk, dv (shapes of q, k, v), dgate (shape of gate,
    or None), dq_norm_w and dk_norm_w ([D]).  Per query head h (kv head g):
        sig = sigmoid(G);  dO = dY * sig;  dG = dY * O * sig * (1 - sig)
        P = softmax(tau q' k'^T over the visible keys)
        dV_g += P^T dO;  dP = dO V^T;  Dr = rowsum(dO * O)
        dS = P * (dP - Dr);  dq' = tau dS K';  dk'_g += tau dS^T Q'
    then back through RoPE (rope_bwd) and RMSNorm (rms_norm_bwd).

    Sampling (for layers too long to differentiate whole): ``rows`` (sorted
    query indices) and/or ``keys`` (sorted key indices) select what is
    returned: dq and dgate at ``rows`` ([B,len(rows),...]), dk and dv at
    ``keys``.  The same per-row steps run, on ``rows`` plus every row that
    sees one of ``keys``; a selected key's gradient sums over exactly the rows
    that see it, so every returned value is the full computation's up to the
    order of the fp64 sums.  The norm-weight gradients sum over all rows and
    are None when sampling.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    tau = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(D)
    pos = pos_offset + np.arange(S, dtype=np.int64)
    sampled = rows is not None or keys is not None
    rsel = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    ksel = np.arange(S) if keys is None else np.asarray(keys, dtype=np.int64)
    # the query rows to run: the selected ones and every row that sees a
    # selected key (rows i with 0 <= i - j < window, or i >= j when global)
    need = np.zeros(S, dtype=bool)
    need[rsel] = True
    if keys is not None:
        for j in ksel:
            need[j:S if window == 0 else min(S, j + window)] = True
    else:
        need[:] = True
    run_rows = np.nonzero(need)[0]
    dq = np.zeros((B, len(rsel), Hq, D))
    dk = np.zeros((B, len(ksel), Hkv, D))
    dv = np.zeros((B, len(ksel), Hkv, D))
    dgate = None if gate is None else np.zeros((B, len(rsel), Hq, D))
    dwq = np.zeros(D)
    dwk = np.zeros(D)
    for b in range(B):
        qp = apply_partial_rope(rms_norm(q[b], q_norm_w, rms_eps), pos, rope_dim, rope_theta)
        kp = apply_partial_rope(rms_norm(k[b], k_norm_w, rms_eps), pos, rope_dim, rope_theta)
        dqp = np.zeros_like(qp)
        dkp = np.zeros_like(kp)
        dvb = np.zeros_like(v[b])
        dgb = None if gate is None else np.zeros((S, Hq, D))
        for c0 in range(0, len(run_rows), chunk):
            ridx = run_rows[c0:c0 + chunk]
            lo = 0 if window == 0 else max(0, int(ridx[0]) - window + 1)
            hi = int(ridx[-1]) + 1
            jj = np.arange(lo, hi)
            mask = visible(ridx[:, None], jj[None, :], window)
            for g in range(Hkv):
                kg = kp[lo:hi, g, :]
                vg = v[b, lo:hi, g, :]
                for hh in range(grp):
                    h = g * grp + hh
                    s = np.where(mask, tau * (qp[ridx, h, :] @ kg.T), -np.inf)
                    e = np.exp(s - np.max(s, axis=1, keepdims=True))
                    P = e / np.sum(e, axis=1, keepdims=True)
                    o = P @ vg
                    dy = dout[b, ridx, h, :]
                    if gate is not None:
                        sg = _sigmoid(np.asarray(gate[b, ridx, h, :], dtype=np.float64))
                        do = dy * sg
                        dgb[ridx, h, :] = dy * o * sg * (1.0 - sg)
                    else:
                        do = dy
                    dvb[lo:hi, g, :] += P.T @ do
                    dP = do @ vg.T
                    dr = np.sum(do * o, axis=1, keepdims=True)
                    dS = P * (dP - dr)
                    dqp[ridx, h, :] += tau * (dS @ kg)
                    dkp[lo:hi, g, :] += tau * (dS.T @ qp[ridx, h, :])
        dqh = rope_bwd(dqp[rsel], pos[rsel], rope_dim, rope_theta)
        dkh = rope_bwd(dkp[ksel], pos[ksel], rope_dim, rope_theta)
        dq[b], gq = rms_norm_bwd(q[b, rsel], q_norm_w, rms_eps, dqh)
        dk[b], gk = rms_norm_bwd(k[b, ksel], k_norm_w, rms_eps, dkh)
        dv[b] = dvb[ksel]
        if dgate is not None:
            dgate[b] = dgb[rsel]
        dwq += gq
        dwk += gk
    return {"dq": dq, "dk": dk, "dv": dv, "dgate": dgate,
            "dq_norm_w": None if sampled else dwq, "dk_norm_w": None if sampled else dwk}


# ---------------------------------------------------------------------------
# The projections on either side of the attention
# ([RB] 核心方法 and [SB] 🏗️ 架构: hidden size 4096, 32 query / 8 KV heads of
# 128 dims; [SB] 🏗️ 架构: the local output is multiplied by a sigmoid gate)
# ---------------------------------------------------------------------------
def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T for a weight stored [out_features, in_features].

    Reading: the pages name the layer sizes only; a bias-free linear map with
    the weight stored output-major is the plainest form of a Transformer
    projection.  x [T, in], w [out, in] -> y [T, out], in float64.
    """
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def qkvg_proj(x: np.ndarray, w: np.ndarray, n_q_heads: int, n_kv_heads: int,
              head_dim: int, gated: bool):
    """The fused input projection of one attention layer.

    Reading: the rows of w stack W_q (n_q_heads * head_dim rows), W_k and
    W_v (n_kv_heads * head_dim rows each) and, on a gated layer, W_g
    (n_q_heads * head_dim rows: the gate has the output's shape, since it
    multiplies the attention output elementwise).  Column h * head_dim + d of
    each part is head h, dim d.  Returns (q [T,Hq,D], k [T,Hkv,D], v, g or
    None).
    """
    y = linear(x, w)
    T = y.shape[0]
    nq, nk = n_q_heads * head_dim, n_kv_heads * head_dim
    assert y.shape[1] == 2 * nq + 2 * nk if gated else nq + 2 * nk
    q = y[:, :nq].reshape(T, n_q_heads, head_dim)
    k = y[:, nq:nq + nk].reshape(T, n_kv_heads, head_dim)
    v = y[:, nq + nk:nq + 2 * nk].reshape(T, n_kv_heads, head_dim)
    g = y[:, nq + 2 * nk:].reshape(T, n_q_heads, head_dim) if gated else None
    return q, k, v, g


# ---------------------------------------------------------------------------
# FP8 (E4M3) matrix multiplies
# ([RB] 前置知识 › FP8 混合精度训练与 TWEO: forward matrix multiplies in E4M3
# with per-tensor scaling factors)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of E4M3 codes (OCP: sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent 0 is subnormal; 0x7F / 0xFF are NaN, there are no
    infinities).  float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0**-9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def quantize_e4m3(x: np.ndarray, scale: float):
    """E4M3 codes and values of x * scale (scale a number, or an array that
    broadcasts against x).

    Reading: the product is formed in float32 (the precision of the kernel
    that takes the decision), then clamped to [-448, 448] and rounded to the
    nearest E4M3 value with ties to even; the sign of a value that rounds to
    zero is kept (negative zero).  Returns (codes uint8, values float64).
    """
    v = (np.asarray(x, dtype=np.float32) * np.asarray(scale, dtype=np.float32)).astype(np.float64)
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    neg = np.signbit(v)
    a = np.abs(v)
    # binade exponent of a (exact: frexp), the subnormal grid below 2^-6
    _, ex = np.frexp(np.maximum(a, 2.0**-6))
    quantum = np.exp2(ex - 1 - 3.0)
    q = np.round(a / quantum) * quantum  # exact scaling; numpy rounds ties to even
    # encode
    _, qex = np.frexp(np.where(q > 0, q, 1.0))
    normal = q >= 2.0**-6
    E = np.where(normal, qex - 1 + 7, 0)
    M = np.where(normal, q / np.exp2(qex - 1.0) * 8 - 8, q / 2.0**-9)
    codes = (np.where(neg, 0x80, 0) | (E.astype(np.int64) << 3) | M.astype(np.int64))
    return codes.astype(np.uint8), np.where(neg, -q, q)


def e4m3_row_scale(x: np.ndarray) -> np.ndarray:
    """Per-row power-of-two scale for quantizing a tensor computed on the fly
    (no amax history exists for it): s = 2^(8 - e) where amax = m 2^e with
    m in [0.5, 1) (frexp; amax = 0 gives e = 0), e clamped to >= -100 so that
    s stays finite in float32.  Then amax * s lies in [128, 256), inside
    E4M3's range, and the scaling itself is exact.  Reading: the pages scale
    per tensor from an amax history; for queries made inside the kernel the
    current amax of each head's row is used."""
    amax = np.max(np.abs(np.asarray(x, dtype=np.float64)), axis=-1)
    _, e = np.frexp(amax)
    return np.exp2(8.0 - np.maximum(e, -100))


def e4m3_rows(x: np.ndarray) -> np.ndarray:
    """Each row of x [G,D] quantized to E4M3 with its ``e4m3_row_scale``;
    returns the values the codes stand for (decode(code) / s)."""
    x = np.asarray(x, dtype=np.float64)
    s = e4m3_row_scale(x)[:, None]
    return quantize_e4m3(x, s)[1] / s


def attention_decode_fp8(q, k_new, v_new, k_codes, v_codes, seq_lens, *, k_scale: float,
                         v_scale: float, ring: bool, window: int, gate, q_norm_w, k_norm_w,
                         rope_dim: int, rope_theta: float, rms_eps: float,
                         softmax_scale: float = 0.0, pos_offset: int = 0,
                         quantize_q: bool = True):
    """Decode against a KV cache stored in E4M3 ([RB] 前置知识 › FP8 混合精度训练与
    TWEO for the format and per-tensor scaling; the cache-size row of [RB]'s
    structured-data table for why the cache is what decode streams).

    k_codes, v_codes uint8 [B,Hkv,cap,D]: codes of K' * k_scale and
    V * v_scale.  Reading: a cached code c stands for e4m3_decode(c) / scale;
    the new token's K' (step 1 of ``decode_group``, in fp64) and V are
    quantized with ``quantize_e4m3`` into their slot; the step is then
    ``decode_group`` over the dequantized cache, with the new token already
    in it.  QK^T is an E4M3 matrix multiply: with ``quantize_q`` each
    head's normalised, rotated query is quantized by ``e4m3_rows`` first
    (products of E4M3 values are exact, so only the sum's rounding remains).
    P V stays in the cache's value precision.  Returns (out [B,Hq,D],
    lse [B,Hq], k_codes_after, v_codes_after).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    grp = Hq // Hkv
    kc = np.array(k_codes, dtype=np.uint8, copy=True)
    vc = np.array(v_codes, dtype=np.uint8, copy=True)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        p = pos_offset + L - 1
        slot = (L - 1) % cap if ring else L - 1
        for g in range(Hkv):
            if k_new is not None:
                kn = rms_norm(np.asarray(k_new[b, g], dtype=np.float64)[None, None, :],
                              k_norm_w, rms_eps)
                kn = apply_partial_rope(kn, np.array([p]), rope_dim, rope_theta)[0, 0]
                kc[b, g, slot] = quantize_e4m3(kn, k_scale)[0]
                vc[b, g, slot] = quantize_e4m3(np.asarray(v_new[b, g]), v_scale)[0]
            hs = slice(g * grp, (g + 1) * grp)
            o, ls, _ = decode_group(
                q[b, hs], None, None, e4m3_decode(kc[b, g]) / k_scale,
                e4m3_decode(vc[b, g]) / v_scale, L, ring=ring, window=window,
                gate_group=None if gate is None else gate[b, hs], q_norm_w=q_norm_w,
                k_norm_w=k_norm_w, rope_dim=rope_dim, rope_theta=rope_theta, rms_eps=rms_eps,
                softmax_scale=softmax_scale, pos_offset=pos_offset,
                q_map=e4m3_rows if quantize_q else None)
            out[b, hs] = o
            lse[b, hs] = ls
    return out, lse, kc, vc


def attention_fwd_fp8(q, k, v, gate, q_norm_w, k_norm_w, *, k_scale: float, window: int,
                      rope_dim: int, rope_theta: float, rms_eps: float,
                      softmax_scale: float = 0.0, pos_offset: int = 0, rows=None,
                      chunk: int = 1024):
    """Prefill / training forward with QK^T as an E4M3 matrix multiply ([RB]
    前置知识 › FP8 混合精度训练与 TWEO: forward matmuls in E4M3 with
    power-of-two scales; [SB] ⚙️ 训练系统: hybrid FP8 training).

    Reading, the same as the E4M3 decode's: the normalised, rotated keys K'
    (in fp64) are quantized with the caller's per-tensor ``k_scale``
    (``quantize_e4m3``: the product formed in float32, clamped to +-448,
    rounded to nearest even) and enter as code / k_scale; each query head's
    normalised, rotated row q' is quantized with its own power-of-two scale
    (``e4m3_rows``).  The scores tau q~' . k~' are then exact up to the
    summation (E4M3 products are exact), and the softmax, P V (V as given, in
    bf16) and the gate are those of ``attention_fwd``.  Returns (out, lse) as
    ``attention_fwd`` does.
    """
    def k_map(kn):
        return quantize_e4m3(kn, k_scale)[1] / k_scale

    def q_map(qn):
        r, h, d = qn.shape
        return e4m3_rows(qn.reshape(r * h, d)).reshape(r, h, d)

    return attention_fwd(q, k, v, gate, q_norm_w, k_norm_w, window=window, rope_dim=rope_dim,
                         rope_theta=rope_theta, rms_eps=rms_eps, softmax_scale=softmax_scale,
                         pos_offset=pos_offset, rows=rows, chunk=chunk, q_map=q_map,
                         k_map=k_map)


# ---------------------------------------------------------------------------
# KV-cache arithmetic and the layer schedule
# ([RB] structured-data table row "256K 上下文推理 KV 缓存"; [SB] 🏗️ 架构)
# ---------------------------------------------------------------------------
def kv_cache_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int,
                             bytes_per_elem: int) -> int:
    """Bytes of K and V cached per token over ``n_layers`` attention layers."""
    return n_layers * n_kv_heads * head_dim * 2 * bytes_per_elem


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int,
                   bytes_per_elem: int, n_tokens: int, batch: int = 1) -> int:
    """Cache bytes for ``batch`` sequences of ``n_tokens`` tokens."""
    return kv_cache_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_elem) \
        * n_tokens * batch


def layer_schedule(n_layers: int = 32, period: int = 6) -> list:
    """Layer kinds, 1-based: every ``period``-th layer is global, the rest
    are gated sliding-window ([RB] 前置知识: global layers 6/12/18/24/30)."""
    return ["global" if (l % period) == 0 else "swa" for l in range(1, n_layers + 1)]


def inband_pairs(S: int, window: int) -> int:
    """Number of visible (query, key) pairs of one head over S rows."""
    if window == 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window
