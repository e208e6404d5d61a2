#!/usr/bin/env python3
"""Benchmark of the ZGCM-1 hybrid attention path on one MI355X.

One step = one forward pass of a 256K-token 5:1 block: five gated
sliding-window (W = 128) layers and one global causal layer, batch 1, GQA
32/8, head dim 128, each layer on its own seeded bf16 N(0,1) inputs (QK-RMSNorm
and partial RoPE on 42 dims run inside the library).  The printed JSON line
reports the block's attention TFLOP/s (in-band pairs only, 512 flop per pair
per query head) and tokens/s, the roofline of the dominant kernel (the global
layer's flash kernel, MFMA-bound), the other workloads as components (gated
SWA B4xS4096, global S16384, one decode step against a 256K cache) and the
fp64 CPU oracle timed on a bounded sample of the same block.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # dense FP8 MFMA, MI355X spec
# The E4M3 attention runs Q K^T (half the flops) at the FP8 rate and P V (the
# other half) at the bf16 rate: at both peaks a layer takes F/2 / 5000 +
# F/2 / 2500 = F / 3333.3 s per TFLOP F.
PEAK_MIXED_FP8_TFLOPS = round(2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS), 1)
# the E4M3 forward's per-tensor K' scale: the keys' RMSNorm bounds |K'| by
# sqrt(128) max|w_k| (about 15 for the benchmark's weights), so 16 stays
# inside E4M3's 448
FP8_K_SCALE = 16.0
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLOP_PER_PAIR = 4 * 128     # QK^T and PV, 2 flop per MAC, head dim 128
BWD_FLOP_PER_PAIR = 10 * 128  # backward: S, dP, dV, dK, dQ products (algorithmic count)
D = 128
KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flash_causal_global_256k_traffic.json")
# sources the flash kernel is compiled from (the traffic summary is keyed by their hash)
FLASH_SRCS = [os.path.join(ROOT, "global_attention_zg_amd", "csrc", f)
              for f in ("flash_causal.hip", "zg_flash_tile.h", "zg_common.h", "zg_lds.h", "zg_queue.h")]


def inband_pairs(S, W):
    if W == 0 or W >= S:
        return S * (S + 1) // 2
    return W * (W + 1) // 2 + (S - W) * W


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev_tensor(torch, key, shape):
    from global_attention_zg_amd import inputs
    n = int(np.prod(shape))
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    flat = out.view(-1)
    step = 1 << 26
    for s0 in range(0, n, step):
        s1 = min(n, s0 + step)
        bits = inputs.normal_bf16_bits(key, n, s0, s1)
        flat[s0:s1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    return out


def norm_w(torch, key):
    from global_attention_zg_amd import inputs
    return torch.from_numpy(inputs.norm_weight(key, D)).cuda()


class Layer:
    """Device-resident inputs, outputs and workspace of one forward layer."""

    def __init__(self, torch, bd, tag, layer, B, S, Hq, Hkv, window, gated, k_scale=None):
        from global_attention_zg_amd import inputs
        self.window = window
        self.k_scale = k_scale  # set: the E4M3 forward with this per-tensor K' scale
        self.q = dev_tensor(torch, (tag, layer, inputs.T_Q), (B, S, Hq, D))
        self.k = dev_tensor(torch, (tag, layer, inputs.T_K), (B, S, Hkv, D))
        self.v = dev_tensor(torch, (tag, layer, inputs.T_V), (B, S, Hkv, D))
        self.g = dev_tensor(torch, (tag, layer, inputs.T_GATE), (B, S, Hq, D)) if gated else None
        self.gq = norm_w(torch, (tag, layer, inputs.T_GQ))
        self.gk = norm_w(torch, (tag, layer, inputs.T_GK))
        self.out = torch.empty_like(self.q)
        p = bd.make_params(B, S, Hq, Hkv, D, window)
        ws = bd.zg_attn_fwd_fp8_workspace_size(p) if k_scale else bd.zg_attn_fwd_workspace_size(p)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.bd = bd
        self.flops = B * Hq * inband_pairs(S, window) * FLOP_PER_PAIR
        self.alg_bytes = (self.q.numel() + self.k.numel() + self.v.numel() + self.out.numel()
                          + (self.g.numel() if gated else 0)) * 2

    def __call__(self):
        if self.k_scale:
            self.bd.zg_attn_fwd_fp8(self.q, self.k, self.v, self.g, self.gq, self.gk,
                                    k_scale=self.k_scale, window=self.window, out=self.out,
                                    workspace=self.ws, **KW)
        else:
            self.bd.zg_attn_fwd(self.q, self.k, self.v, self.g, self.gq, self.gk,
                                window=self.window, out=self.out, workspace=self.ws, **KW)


class BwdLayer:
    """A forward layer plus what its training backward reads and writes."""

    def __init__(self, torch, bd, tag, B, S, Hq, Hkv, window, gated):
        from global_attention_zg_amd import inputs
        self.f = Layer(torch, bd, tag, 0, B, S, Hq, Hkv, window, gated)
        f = self.f
        self.dout = dev_tensor(torch, (tag, 0, inputs.T_DOUT), (B, S, Hq, D))
        self.lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        bd.zg_attn_fwd(f.q, f.k, f.v, f.g, f.gq, f.gk, window=window, out=f.out, lse=self.lse,
                       workspace=f.ws, **KW)
        self.grads = dict(dq=torch.empty_like(f.q), dk=torch.empty_like(f.k),
                          dv=torch.empty_like(f.v),
                          dgate=None if f.g is None else torch.empty_like(f.g),
                          dq_norm_w=torch.empty(D, dtype=torch.float32, device="cuda"),
                          dk_norm_w=torch.empty(D, dtype=torch.float32, device="cuda"))
        p = bd.make_params(B, S, Hq, Hkv, D, window)
        self.ws = torch.empty(bd.zg_attn_bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
        self.bd = bd
        self.flops = B * Hq * inband_pairs(S, window) * BWD_FLOP_PER_PAIR
        nq = f.q.numel() * (4 + (2 if gated else 0))  # q, out, dout, dq (+ gate, dgate)
        nk = f.k.numel() * 4                           # k, v, dk, dv
        self.alg_bytes = (nq + nk) * 2 + self.lse.numel() * 4

    def __call__(self):
        f = self.f
        self.bd.zg_attn_bwd(f.q, f.k, f.v, f.g, f.gq, f.gk, f.out, self.lse, self.dout,
                            window=f.window, workspace=self.ws, **self.grads, **KW)


WARM_S = 0.1


def warm_up(torch, fn, seconds=WARM_S):
    """Run fn back to back, in batches of 8 between synchronisations, for
    about `seconds`: the timed calls that follow then run at the clock of
    sustained work.  After an idle spell the GPU takes ~15 calls of a 2 ms
    kernel to come back up to speed, which a few warm-up calls would leave
    inside the timed region."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_events(torch, fn, iters):
    """Average duration of fn() on the current stream, by HIP events, after
    warm_up."""
    warm_up(torch, fn)
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3


def time_stats(torch, fn, iters, flush=None):
    """Median, min and max duration of fn() by HIP events on the current
    stream. With `flush` (a device buffer larger than L2 plus the MALL), the
    buffer is rewritten before every timed call, outside the events, so that
    each call starts with cold caches.  warm_up runs first."""
    warm_up(torch, fn)
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        if flush is not None:
            flush.fill_(i & 0xFF)
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    ts = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
    return float(np.median(ts)), float(ts.min()), float(ts.max())


def flush_buffer(torch):
    """512 MiB of device memory: twice the MALL, far more than the L2s."""
    return torch.empty(512 << 20, dtype=torch.uint8, device="cuda")


def flash_source_hash():
    """sha256[:16] of the kernel's sources with their // comments and blank
    lines removed, so that an edit of the comments alone keeps the counters."""
    h = hashlib.sha256()
    for path in FLASH_SRCS:
        with open(path, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the global-layer causal kernel from the committed
    rocprofv3 counter summary, or None if it is missing or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != flash_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def sclk_mhz():
    """Current shader clock of GPU 0 as rocm-smi reports it, or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        for k, v in card.items():
            if "sclk" in k.lower() and "speed" in k.lower():
                return float(str(v).strip("()").lower().replace("mhz", ""))
    except (OSError, ValueError, StopIteration, subprocess.SubprocessError, AttributeError):
        return None
    return None


def reference_peaks(torch, iters=20):
    """Measured ceilings on this GPU beside the published ones: a plain 1 GiB
    device copy (read + write bytes per second), the library bf16 GEMM behind
    torch.mm on 8192^3, and the shader clock."""
    log("reference peaks: 1 GiB copy, 8192^3 bf16 library GEMM")
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    t_copy = time_events(torch, lambda: dst.copy_(src), iters)
    del src, dst
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((m, m), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.mm(a, b, out=c)
    t_mm = time_events(torch, lambda: torch.mm(a, b, out=c), iters)
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * n / t_copy / 1e9, 1),
            "copy_frac_of_spec": round(2 * n / t_copy / 1e9 / PEAK_HBM_GBS, 4),
            "library_gemm_bf16_tflops": round(2.0 * m ** 3 / t_mm / 1e12, 1),
            "library_gemm_frac_of_spec": round(2.0 * m ** 3 / t_mm / 1e12 / PEAK_BF16_TFLOPS, 4),
            "sclk_mhz_after": sclk_mhz(),
            "spec": {"hbm_gbs": PEAK_HBM_GBS, "bf16_tflops": PEAK_BF16_TFLOPS,
                     "sclk_mhz": 2400.0}}


# The global layer's rows the oracle checks and times at 256K: the fixed rows
# of the workload's plan plus 55 seeded ones.
# leading rows of one gated SWA layer of the 256K block in the oracle sample
SWA_SAMPLE_ROWS = 32768


def host_info():
    """CPU model, cores this process may use, and the BLAS thread count."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas}


def _f64_rows(key, S, H, rows):
    """Rows `rows` of a seeded [1, S, H, D] bf16 tensor as float64 [1, len(rows), H, D]."""
    from global_attention_zg_amd import inputs
    from oracle import zg_oracle as orc
    total, per = S * H * D, H * D
    out = np.empty((1, len(rows), H, D))
    for i, r in enumerate(rows):
        bits = inputs.normal_bf16_bits(key, total, r * per, (r + 1) * per)
        out[0, i] = orc.bf16_bits_to_f64(bits).reshape(H, D)
    return out


def _f64_prefix(key, S, H, n):
    """The first n positions of a seeded [1, S, H, D] bf16 tensor, float64."""
    from global_attention_zg_amd import inputs
    from oracle import zg_oracle as orc
    return orc.bf16_bits_to_f64(inputs.normal_bf16_bits(key, S * H * D, 0, n * H * D)).reshape(
        1, n, H, D)


def cpu_baseline(gpu_rows=None):
    """The fp64 oracle, as it stands, timed on the host on each workload:
    in full where that takes a few seconds, otherwise on a stated sample whose
    time is scaled to the whole workload by its share of the (query, key)
    pairs (labelled extrapolated).  Inputs are the benchmark's own seeded
    tensors.  Only the oracle calls are timed, not the input generation.

    `gpu_rows` (name -> the timed run's output on the sampled rows) is
    compared with the oracle's rows of the 256K block: causal rows depend only
    on the keys before them, so rows of the full layers can be checked one by
    one."""
    from global_attention_zg_amd import inputs
    from oracle import zg_oracle as orc

    gq4 = lambda t, l: inputs.norm_weight((t, l, inputs.T_GQ), D).astype(np.float64)  # noqa: E731
    gk4 = lambda t, l: inputs.norm_weight((t, l, inputs.T_GK), D).astype(np.float64)  # noqa: E731
    per_cfg = {}
    parity = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    def record(name, flops_sample, t, flops_full, sample):
        e = {"tflops": round(flops_sample / t / 1e12, 6), "seconds_sample": round(t, 3),
             "sample": sample}
        if flops_sample < flops_full:
            e["seconds_full_extrapolated"] = round(t * flops_full / flops_sample, 2)
            e["kind"] = "sampled, extrapolated by pair count"
        else:
            e["kind"] = "full"
        per_cfg[name] = e

    # tiny pair: B1 S512 4/1 heads, gated SWA and global on the same inputs, in full
    from tests import zg_cases as zc
    c = zc.fwd_case(1, 1, 512, 4, 1, gated=True)
    args = [zc.f64(c[n]) for n in ("q", "k", "v", "gate")]
    w = (c["gq"].astype(np.float64), c["gk"].astype(np.float64))
    _, t1 = timed(lambda: orc.attention_fwd(*args, *w, window=128, **KW))
    _, t2 = timed(lambda: orc.attention_fwd(*args[:3], None, *w, window=0, **KW))
    fl = 4 * (inband_pairs(512, 128) + inband_pairs(512, 0)) * FLOP_PER_PAIR
    record("tiny_pair_s512", fl, t1 + t2, fl, "both layers in full")

    # gated SWA B4 S4096 32/8, in full
    S = 4096
    q = _f64_prefix((2, 0, inputs.T_Q), 4 * S, 32, 4 * S).reshape(4, S, 32, D)
    k = _f64_prefix((2, 0, inputs.T_K), 4 * S, 8, 4 * S).reshape(4, S, 8, D)
    v = _f64_prefix((2, 0, inputs.T_V), 4 * S, 8, 4 * S).reshape(4, S, 8, D)
    g = _f64_prefix((2, 0, inputs.T_GATE), 4 * S, 32, 4 * S).reshape(4, S, 32, D)
    _, t = timed(lambda: orc.attention_fwd(q, k, v, g, gq4(2, 0), gk4(2, 0), window=128, **KW))
    fl = 4 * 32 * inband_pairs(S, 128) * FLOP_PER_PAIR
    record("swa_4k_b4", fl, t, fl, "all 4 sequences in full, all 32 heads")

    # global S16384: 64 sampled rows, all 32 heads
    S = 16384
    rows = inputs.global_sample_rows(S, 55, S)
    q = _f64_rows((3, 0, inputs.T_Q), S, 32, rows)
    k = _f64_prefix((3, 0, inputs.T_K), S, 8, S)
    v = _f64_prefix((3, 0, inputs.T_V), S, 8, S)
    qfull = np.zeros((1, S, 32, D))
    qfull[0, rows] = q[0]
    _, t = timed(lambda: orc.attention_fwd(qfull, k, v, None, gq4(3, 0), gk4(3, 0), window=0,
                                           rows=rows, **KW))
    record("global_16k", 32 * sum(r + 1 for r in rows) * FLOP_PER_PAIR, t,
           32 * inband_pairs(S, 0) * FLOP_PER_PAIR, f"{len(rows)} sampled rows, all 32 heads")
    del q, k, v, qfull

    # the 256K block: one gated SWA layer's first SWA_SAMPLE_ROWS rows (x5 layers)
    # and the global layer's 64 sampled rows
    S = 262144
    n = SWA_SAMPLE_ROWS
    q = _f64_prefix((4, 0, inputs.T_Q), S, 32, n)
    k = _f64_prefix((4, 0, inputs.T_K), S, 8, n)
    v = _f64_prefix((4, 0, inputs.T_V), S, 8, n)
    g = _f64_prefix((4, 0, inputs.T_GATE), S, 32, n)
    (ref_swa, _), t_swa = timed(lambda: orc.attention_fwd(q, k, v, g, gq4(4, 0), gk4(4, 0),
                                                          window=128, **KW))
    del q, k, v, g
    rows = inputs.global_sample_rows(S)
    qs = _f64_rows((4, 5, inputs.T_Q), S, 32, rows)
    k = _f64_prefix((4, 5, inputs.T_K), S, 8, S)
    v = _f64_prefix((4, 5, inputs.T_V), S, 8, S)

    # q with only the sampled rows written: the oracle reads just those rows
    # (np.zeros maps untouched pages lazily, so this holds 64 rows of memory)
    qfull = np.zeros((1, S, 32, D))
    qfull[0, rows] = qs[0]
    (ref_glob, _), t_glob = timed(lambda: orc.attention_fwd(qfull, k, v, None, gq4(4, 5),
                                                            gk4(4, 5), window=0, rows=rows,
                                                            **KW))
    del k, v, qfull
    fl_swa = 32 * inband_pairs(n, 128) * FLOP_PER_PAIR
    fl_glob = 32 * sum(r + 1 for r in rows) * FLOP_PER_PAIR
    full_block = (5 * 32 * inband_pairs(S, 128) + 32 * inband_pairs(S, 0)) * FLOP_PER_PAIR
    # the block time: five SWA layers scaled from the prefix, the global layer from the rows
    t_block = 5 * t_swa * inband_pairs(S, 128) / inband_pairs(n, 128) + \
        t_glob * 32 * inband_pairs(S, 0) * FLOP_PER_PAIR / fl_glob
    per_cfg["block_256k"] = {
        "tflops": round((fl_swa + fl_glob) / (t_swa + t_glob) / 1e12, 6),
        "seconds_sample": round(t_swa + t_glob, 3),
        "seconds_full_extrapolated": round(t_block, 1),
        "kind": "sampled, extrapolated by pair count",
        "sample": f"first {n} rows of one gated SWA layer (x5 layers) and {len(rows)} sampled "
                  "rows of the global layer, all 32 heads"}
    if gpu_rows is not None:
        for name, ref, what in (("swa_layer0", ref_swa, f"rows 0..{n - 1}"),
                                ("global_layer5", ref_glob,
                                 f"{len(rows)} rows: {list(inputs.GLOBAL_ROWS_FIXED)} + 55 seeded")):
            d = gpu_rows[name] - ref
            parity[name] = {"rows": what + ", all 32 heads", "max_abs": float(np.abs(d).max()),
                            "rel_rms": float(np.sqrt((d * d).sum() / (ref * ref).sum())),
                            "bound": "max_abs <= 2e-2 and rel_rms <= 1e-2"}

    # decode at 256K, B16: one (sequence, KV head) group of the global cache
    # per sequence (16 of 128), and the SWA ring in full
    B, Hq, Hkv, L = 16, 32, 8, 262145
    grp = Hq // Hkv
    tq = 0.0
    pairs = [(b, b % Hkv) for b in range(B)]
    for b, gi in pairs:
        def slab(t):
            per = L * D
            s0 = (b * Hkv + gi) * per
            return orc.bf16_bits_to_f64(inputs.normal_bf16_bits((5, 0, t), B * Hkv * per, s0,
                                                                s0 + per)).reshape(L, D)
        kc, vc = slab(inputs.T_KCACHE), slab(inputs.T_VCACHE)
        qg = orc.bf16_bits_to_f64(zc.bits((5, 0, inputs.T_Q), (B, Hq, D))[b, gi * grp:(gi + 1) * grp])
        kn = orc.bf16_bits_to_f64(zc.bits((5, 0, inputs.T_KNEW), (B, Hkv, D))[b, gi])
        vn = orc.bf16_bits_to_f64(zc.bits((5, 0, inputs.T_VNEW), (B, Hkv, D))[b, gi])
        _, t = timed(lambda: orc.decode_group(qg, kn, vn, kc, vc, L, ring=False, window=0,
                                              gate_group=None, q_norm_w=gq4(5, 0),
                                              k_norm_w=gk4(5, 0), **KW))
        tq += t
    record("decode_global_256k", len(pairs) * grp * L * FLOP_PER_PAIR, tq,
           B * Hq * L * FLOP_PER_PAIR,
           f"{len(pairs)} of the 128 (sequence, KV head) groups, one per sequence, 262145 keys each")
    qb = zc.bits((5, 1, inputs.T_Q), (B, Hq, D))
    kcb = zc.bits((5, 1, inputs.T_KCACHE), (B, Hkv, 128, D))
    vcb = zc.bits((5, 1, inputs.T_VCACHE), (B, Hkv, 128, D))
    knb = zc.bits((5, 1, inputs.T_KNEW), (B, Hkv, D))
    vnb = zc.bits((5, 1, inputs.T_VNEW), (B, Hkv, D))
    gb = zc.bits((5, 1, inputs.T_GATE), (B, Hq, D))
    _, t = timed(lambda: orc.attention_decode(zc.f64(qb), zc.f64(knb), zc.f64(vnb), zc.f64(kcb),
                                              zc.f64(vcb), [L] * B, ring=True, window=128,
                                              gate=zc.f64(gb), q_norm_w=gq4(5, 1),
                                              k_norm_w=gk4(5, 1), **KW))
    fl = B * Hq * 128 * FLOP_PER_PAIR
    record("decode_swa_ring", fl, t, fl, "all 16 sequences, ring of 128")

    info = host_info()
    head = per_cfg["block_256k"]
    return dict(value=head["tflops"], unit="TFLOP/s", cores=info["blas_threads"] or
                info["affinity_cores"], kind="oracle",
                sample=head["sample"] + f"; fp64 numpy, {head['seconds_sample']} s on the host",
                seconds=head["seconds_sample"],
                block_seconds_full_extrapolated=head["seconds_full_extrapolated"],
                per_config=per_cfg, host=info), parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only",
                    choices=["swa4k", "global16k", "decode", "decode_block", "block_global", "bwd",
                             "varlen", "proj", "variants", "block_swa", "block_global_fp8"],
                    default=None, help="time one workload only (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only: first run a plain 1 GiB device copy, the reference "
                         "for scaling the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from global_attention_zg_amd import binding as bd
    torch.cuda.set_device(0)
    if args.only:
        if args.copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps({"only": args.only, "components": run_components(torch, bd, args.only,
                                                                          args.steps)}))
        return

    # ---- the 256K 5:1 block: five gated SWA layers + one global layer
    S, B, Hq, Hkv = 262144, 1, 32, 8
    log("generating the 256K block inputs (6 layers)")
    layers = [Layer(torch, bd, 4, l, B, S, Hq, Hkv, 128, True) for l in range(5)]
    layers.append(Layer(torch, bd, 4, 5, B, S, Hq, Hkv, 0, False))
    glob = layers[-1]
    block_flops = sum(l.flops for l in layers)

    def step(ev=None):
        for l in layers[:5]:
            l()
        if ev is not None:
            ev[0].record()
        glob()
        if ev is not None:
            ev[1].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(gevs[i])
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    t_glob = float(np.mean([a.elapsed_time(b) for a, b in gevs])) * 1e-3
    log(f"step {t_step * 1e3:.2f} ms, global layer {t_glob * 1e3:.2f} ms")
    swa_t = time_events(torch, layers[0], 5)
    achieved = glob.flops / t_glob / 1e12
    traffic = read_traffic()

    result = {
        "metric": "attention TFLOP/s & tokens/s per MI355X, gated SWA-128 + global, 4K-256K",
        "value": round(block_flops / t_step / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded bf16 N(0,1) q/k/v/gate per layer, RMSNorm weights 1+0.1N(0,1)",
        "config": {"workload": "zgcm1_5to1_block_prefill_256k", "global_batch": B, "seq_len": S,
                   "layers": "5 gated SWA (W=128) + 1 global causal", "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "rope_dim": 42, "parallelism": "none"},
        "tokens_per_s": round(B * S / t_step, 1),
        "roofline": {"bound": "mfma", "kernel": "flash_causal_kernel (global causal, S=262144)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "block_breakdown_ms": {"swa_layer": round(swa_t * 1e3, 3),
                               "global_layer": round(t_glob * 1e3, 3)},
    }
    # the kernel's output on the rows the oracle sample covers
    from global_attention_zg_amd import inputs
    grow = torch.tensor(inputs.global_sample_rows(S), dtype=torch.long, device="cuda")
    gpu_rows = {"swa_layer0": layers[0].out[:, :SWA_SAMPLE_ROWS].float().cpu().numpy().astype(
                    np.float64),
                "global_layer5": layers[5].out[:, grow].float().cpu().numpy().astype(np.float64)}
    del layers, glob
    torch.cuda.empty_cache()

    if not args.no_components:
        result["components"] = run_components(torch, bd, None, 20)
        result["reference_peaks"] = reference_peaks(torch)

    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle, bounded sample)")
        result["cpu_baseline"], result["parity_vs_oracle"] = cpu_baseline(gpu_rows)
    result["host"] = host_info()
    print(json.dumps(result), flush=True)


def run_components(torch, bd, only, iters):
    """Per-workload timings: gated SWA B4xS4096, global S16384, decode at 256K."""
    comps = {}
    if only in (None, "swa4k"):
        log("component: gated SWA B4 S4096")
        l2 = Layer(torch, bd, 2, 0, 4, 4096, 32, 8, 128, True)
        for _ in range(3):
            l2()
        fl = flush_buffer(torch)
        t, t_lo, t_hi = time_stats(torch, l2, iters, flush=fl)
        comps["swa_4k_b4"] = {"ms": round(t * 1e3, 4), "ms_min": round(t_lo * 1e3, 4),
                              "ms_max": round(t_hi * 1e3, 4), "caches_flushed": True,
                              "tflops": round(l2.flops / t / 1e12, 2),
                              "tokens_per_s": round(4 * 4096 / t, 1),
                              "hbm_gbs_alg": round(l2.alg_bytes / t / 1e9, 1),
                              "frac_hbm": round(l2.alg_bytes / t / 1e9 / PEAK_HBM_GBS, 4)}
        t_warm = time_events(torch, l2, iters)
        comps["swa_4k_b4"]["ms_mean_warm_caches"] = round(t_warm * 1e3, 4)
        del l2, fl
    if only in (None, "global16k"):
        log("component: global S16384")
        l3 = Layer(torch, bd, 3, 0, 1, 16384, 32, 8, 0, False)
        for _ in range(2):
            l3()
        t, t_lo, t_hi = time_stats(torch, l3, max(1, iters // 2))
        comps["global_16k"] = {"ms": round(t * 1e3, 4), "ms_min": round(t_lo * 1e3, 4),
                               "ms_max": round(t_hi * 1e3, 4),
                               "tflops": round(l3.flops / t / 1e12, 2),
                               "tokens_per_s": round(16384 / t, 1),
                               "frac_mfma": round(l3.flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del l3
        # the E4M3 variant on the same inputs: half the flops (Q K^T) at the
        # FP8 peak, half (P V) at the bf16 peak
        l8 = Layer(torch, bd, 3, 0, 1, 16384, 32, 8, 0, False, k_scale=FP8_K_SCALE)
        for _ in range(2):
            l8()
        t8, t8_lo, t8_hi = time_stats(torch, l8, max(1, iters // 2))
        comps["global_16k_fp8"] = {"ms": round(t8 * 1e3, 4), "ms_min": round(t8_lo * 1e3, 4),
                                   "ms_max": round(t8_hi * 1e3, 4), "k_scale": FP8_K_SCALE,
                                   "tflops": round(l8.flops / t8 / 1e12, 2),
                                   "tokens_per_s": round(16384 / t8, 1),
                                   "peak_mixed_tflops": PEAK_MIXED_FP8_TFLOPS,
                                   "frac_mixed_peak": round(l8.flops / t8 / 1e12 /
                                                            PEAK_MIXED_FP8_TFLOPS, 4),
                                   "speedup_vs_bf16": round(t / t8, 3)}
        del l8
    torch.cuda.empty_cache()
    if only in (None, "decode"):
        comps.update(decode_components(torch, bd, max(1, iters // 2)))
    if only in (None, "decode", "decode_block"):
        comps.update(decode_block_components(torch, bd, max(1, iters // 2)))
    if only in (None, "variants"):
        comps.update(variant_components(torch, bd, max(1, iters // 2)))
    if only in (None, "proj"):
        comps.update(proj_components(torch, bd, max(1, iters // 2)))
    if only in (None, "varlen"):
        comps.update(varlen_components(torch, bd, max(1, iters // 2)))
    if only in (None, "bwd"):
        comps.update(bwd_components(torch, bd, max(1, iters // 2)))
    if only == "block_swa":
        log("gated SWA layer of the 256K block")
        ls = Layer(torch, bd, 4, 0, 1, 262144, 32, 8, 128, True)
        ls()
        t = time_events(torch, ls, max(1, iters // 2))
        comps["block_swa_256k"] = {"ms": round(t * 1e3, 4),
                                   "hbm_gbs_alg": round(ls.alg_bytes / t / 1e9, 1),
                                   "frac_hbm": round(ls.alg_bytes / t / 1e9 / PEAK_HBM_GBS, 4)}
        del ls
    if only == "block_global_fp8":
        log("global layer of the 256K block, E4M3 scores")
        lg = Layer(torch, bd, 4, 5, 1, 262144, 32, 8, 0, False, k_scale=FP8_K_SCALE)
        lg()
        t = time_events(torch, lg, max(1, iters // 2))
        comps["block_global_256k_fp8"] = {"ms": round(t * 1e3, 3),
                                          "tflops": round(lg.flops / t / 1e12, 2),
                                          "frac_mixed_peak": round(lg.flops / t / 1e12 /
                                                                   PEAK_MIXED_FP8_TFLOPS, 4)}
        del lg
    if only == "block_global":
        log("global layer of the 256K block")
        lg = Layer(torch, bd, 4, 5, 1, 262144, 32, 8, 0, False)
        lg()
        t = time_events(torch, lg, max(1, iters // 2))
        comps["block_global_256k"] = {"ms": round(t * 1e3, 3),
                                      "tflops": round(lg.flops / t / 1e12, 2)}
        del lg
    return comps


class DecodeLayer:
    """One layer's decode step, B16 at one new token per sequence: a gated
    SWA layer against its 128-slot ring, or the global layer against a cache
    of `cap` keys."""

    def __init__(self, torch, bd, tag, layer, L, swa):
        from global_attention_zg_amd import inputs
        B, Hq, Hkv = 16, 32, 8
        self.cap, self.ring, self.window = (128, True, 128) if swa else (L, False, 0)
        key = lambda t: (tag, layer, t)  # noqa: E731
        self.kc = dev_tensor(torch, key(inputs.T_KCACHE), (B, Hkv, self.cap, D))
        self.vc = dev_tensor(torch, key(inputs.T_VCACHE), (B, Hkv, self.cap, D))
        self.q = dev_tensor(torch, key(inputs.T_Q), (B, Hq, D))
        self.kn = dev_tensor(torch, key(inputs.T_KNEW), (B, Hkv, D))
        self.vn = dev_tensor(torch, key(inputs.T_VNEW), (B, Hkv, D))
        self.g = dev_tensor(torch, key(inputs.T_GATE), (B, Hq, D)) if swa else None
        self.gq = norm_w(torch, key(inputs.T_GQ))
        self.gk = norm_w(torch, key(inputs.T_GK))
        self.sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        p = bd.make_params(B, 0, Hq, Hkv, D, self.window)
        self.ws = torch.empty(max(16, bd.zg_attn_decode_workspace_size(p, self.cap, 0)),
                              dtype=torch.uint8, device="cuda")
        self.bd = bd

    def __call__(self):
        self.bd.zg_attn_decode(self.q, self.kn, self.vn, self.kc, self.vc, self.sl,
                               ring=self.ring, window=self.window, gate=self.g,
                               q_norm_w=self.gq, k_norm_w=self.gk, out=self.out,
                               workspace=self.ws, **KW)


def decode_block_components(torch, bd, iters):
    """One decode step of a whole 5:1 block (five gated SWA layers, then the
    global layer), B16, issued eagerly and replayed from a captured HIP graph
    (the same six launches sequences without host overhead), at a 256K and a
    4K context."""
    out = {}
    for kind, L in (("decode_block_256k", 262145), ("decode_block_4k", 4097)):
        log(f"component: {kind}")
        layers = [DecodeLayer(torch, bd, 10, i, L, swa=(i < 5)) for i in range(6)]

        def step():
            for layer in layers:
                layer()

        for _ in range(2):
            step()
        t_eager = time_events(torch, step, iters)
        ref = [layer.out.clone() for layer in layers]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a.view(torch.int16), layer.out.view(torch.int16))
                   for a, layer in zip(ref, layers))
        t_graph = time_events(torch, graph.replay, iters)
        keys = 16 * 8 * (L + 5 * 128)
        alg = keys * D * 2 * 2
        # the same step as one launch (zg_attn_decode_block), eager and graphed
        blk = [dict(q=l.q, k_new=l.kn, v_new=l.vn, k_cache=l.kc, v_cache=l.vc, gate=l.g,
                    q_norm_w=l.gq, k_norm_w=l.gk, out=torch.empty_like(l.q), ring=l.ring,
                    window=l.window) for l in layers]
        arr, _ = bd._block_layers(blk, layers[0].sl)
        p = bd.make_params(16, 0, 32, 8, D, 0, **KW)
        ws = torch.zeros(bd.zg_attn_decode_block_workspace_size(p, arr), dtype=torch.uint8,
                         device="cuda")

        def fused():
            bd.zg_attn_decode_block(blk, layers[0].sl, workspace=ws, **KW)

        for _ in range(2):
            fused()
        torch.cuda.synchronize()
        # (the one-launch step splits the global layer differently, so its
        # outputs differ from the per-layer calls' by rounding only)
        fused_diff = max(float((a.float() - d["out"].float()).abs().max().item())
                         for a, d in zip(ref, blk))
        t_fused = time_events(torch, fused, iters)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fused()
        torch.cuda.current_stream().wait_stream(side)
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            fused()
        g2.replay()
        torch.cuda.synchronize()
        t_fused_graph = time_events(torch, g2.replay, iters)
        out[kind] = {"ms_eager": round(t_eager * 1e3, 4), "ms_graph": round(t_graph * 1e3, 4),
                     "tokens_per_s_graph": round(16 / t_graph, 1),
                     "hbm_gbs_alg_graph": round(alg / t_graph / 1e9, 1),
                     "graph_equals_eager": bool(same),
                     "one_launch": {"ms_eager": round(t_fused * 1e3, 4),
                                    "ms_graph": round(t_fused_graph * 1e3, 4),
                                    "tokens_per_s_graph": round(16 / t_fused_graph, 1),
                                    "hbm_gbs_alg_graph": round(alg / t_fused_graph / 1e9, 1),
                                    "max_abs_vs_per_layer_calls": round(fused_diff, 6),
                                    "splits_global": bd.zg_attn_decode_block_num_splits(p, L)}}
        del graph, g2, layers, blk
        torch.cuda.empty_cache()
    return out


def variant_components(torch, bd, iters):
    """The ablation's other configurations: the 1:1 / 3:1 / 5:1 interleave
    arms and full attention over the 32 attention layers at 64K tokens
    (composed from the measured time of one gated SWA layer and one global
    layer at that length), and sliding windows other than 128 (B4 S4096)."""
    out = {}
    S = 65536
    log("component: variants (64K layers)")
    times = {}
    for kind, window, gated in (("swa", 128, True), ("global", 0, False)):
        l = Layer(torch, bd, 12, 0 if gated else 1, 1, S, 32, 8, window, gated)
        for _ in range(2):
            l()
        times[kind] = time_events(torch, l, iters)
        del l
        torch.cuda.empty_cache()
    arms = {}
    for name, period in (("1:1", 2), ("3:1", 4), ("5:1", 6), ("full", 1)):
        n_global = 32 // period
        t = (32 - n_global) * times["swa"] + n_global * times["global"]
        arms[name] = {"global_layers": n_global, "ms_32_layers": round(t * 1e3, 3),
                      "tokens_per_s": round(S / t, 1)}
    for name in ("1:1", "3:1", "5:1"):
        arms[name]["speedup_vs_full"] = round(arms["full"]["ms_32_layers"] /
                                              arms[name]["ms_32_layers"], 3)
    out["interleave_arms_64k"] = {"swa_layer_ms": round(times["swa"] * 1e3, 4),
                                  "global_layer_ms": round(times["global"] * 1e3, 4),
                                  "composed": "each arm's ms_32_layers is the layer counts times "
                                              "the two measured layer times, not a timed run",
                                  "arms": arms}
    for W in (64, 256, 512, 1024):
        log(f"component: swa W{W} B4 S4096")
        l = Layer(torch, bd, 13, W, 4, 4096, 32, 8, W, True)
        for _ in range(2):
            l()
        t = time_events(torch, l, iters)
        out[f"swa_w{W}_4k_b4"] = {"ms": round(t * 1e3, 4), "tflops": round(l.flops / t / 1e12, 2),
                                  "hbm_gbs_alg": round(l.alg_bytes / t / 1e9, 1),
                                  "frac_hbm": round(l.alg_bytes / t / 1e9 / PEAK_HBM_GBS, 4),
                                  "frac_mfma": round(l.flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del l
    torch.cuda.empty_cache()
    return out


def proj_components(torch, bd, iters):
    """The projections around the attention at the model's sizes (hidden
    4096, 32/8 heads of 128): the gated layer's fused q/k/v/gate input
    projection (N 10240) and the output projection (N 4096), at 16K and 64K
    tokens."""
    from global_attention_zg_amd import inputs
    out = {}
    hidden, Hq, Hkv = 4096, 32, 8
    for T in (16384, 65536):
        x = dev_tensor(torch, (11, T, inputs.T_X), (T, hidden))
        for kind, N in (("qkvg", 2 * Hkv * D + 2 * Hq * D), ("o", hidden)):
            name = f"proj_{kind}_{T // 1024}k"
            log(f"component: {name}")
            w = dev_tensor(torch, (11, N, inputs.T_W), (N, hidden))
            if kind == "qkvg":
                q = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
                k = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device="cuda")
                v = torch.empty_like(k)
                g = torch.empty_like(q)
                fn = lambda: bd.zg_qkvg_proj(x, w, Hq, Hkv, True, q=q, k=k, v=v,  # noqa: E731
                                             gate=g)
            else:
                y = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
                fn = lambda: bd.zg_linear(x, w, out=y)  # noqa: E731
            for _ in range(2):
                fn()
            t = time_events(torch, fn, iters)
            flops = 2.0 * T * N * hidden
            out[name] = {"ms": round(t * 1e3, 4), "tflops": round(flops / t / 1e12, 1),
                         "frac_mfma": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "M": T, "N": N, "K": hidden}
            # the same product with E4M3 operands (per-tensor scales; the
            # weight quantized once, the activations per call)
            log(f"component: {name}_fp8")
            wq = bd.zg_quantize_fp8(w, 32.0 * hidden ** 0.5)
            xq = torch.empty((T, hidden), dtype=torch.uint8, device="cuda")
            yq = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
            osc = 1.0 / (32.0 * 32.0 * hidden ** 0.5)
            fq = lambda: bd.zg_linear_fp8(xq, wq, osc, out=yq)  # noqa: E731
            fz = lambda: bd.zg_quantize_fp8(x, 32.0, out=xq)  # noqa: E731
            fz()
            for _ in range(2):
                fq()
            tq = time_events(torch, fq, iters)
            tz = time_events(torch, fz, iters)
            out[name + "_fp8"] = {"ms": round(tq * 1e3, 4), "tflops": round(flops / tq / 1e12, 1),
                                  "frac_fp8_mfma": round(flops / tq / 1e12 / PEAK_FP8_TFLOPS, 4),
                                  "quantize_x_ms": round(tz * 1e3, 4),
                                  "M": T, "N": N, "K": hidden}
            del w, wq, xq, yq
        del x
        torch.cuda.empty_cache()
    return out


VARLEN_LENS_SEED = 9


def varlen_components(torch, bd, iters):
    """A packed serving batch: 16 prompts of seeded lengths in 1..8192, 32/8
    heads, through the gated SWA layer and the global layer."""
    from global_attention_zg_amd import inputs
    lens = [int(x) for x in np.random.default_rng(VARLEN_LENS_SEED).integers(1, 8193, size=16)]
    T = sum(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    q = dev_tensor(torch, (8, 0, inputs.T_Q), (T, 32, D))
    k = dev_tensor(torch, (8, 0, inputs.T_K), (T, 8, D))
    v = dev_tensor(torch, (8, 0, inputs.T_V), (T, 8, D))
    g = dev_tensor(torch, (8, 0, inputs.T_GATE), (T, 32, D))
    gq = norm_w(torch, (8, 0, inputs.T_GQ))
    gk = norm_w(torch, (8, 0, inputs.T_GK))
    o = torch.empty_like(q)
    # sized for the global layer (K' and the causal kernel's queue counters)
    ws_p = bd.make_params(len(lens), max(lens), 32, 8, D, 0)
    ws = torch.empty(bd.zg_attn_fwd_varlen_workspace_size(ws_p, T), dtype=torch.uint8,
                     device="cuda")
    out = {}
    for kind, window, gate in (("varlen_swa_16x", 128, g), ("varlen_global_16x", 0, None)):
        log(f"component: {kind}")

        def fn():
            bd.zg_attn_fwd_varlen(q, k, v, gate, gq, gk, cu, max(lens), window=window, out=o,
                                  workspace=ws, **KW)

        for _ in range(2):
            fn()
        t = time_events(torch, fn, iters)
        flops = 32 * sum(inband_pairs(n, window) for n in lens) * FLOP_PER_PAIR
        r = {"ms": round(t * 1e3, 4), "tokens": T, "tokens_per_s": round(T / t, 1),
             "tflops": round(flops / t / 1e12, 2)}
        if window:
            alg = (q.numel() * 3 + k.numel() * 2) * 2  # q, gate, out, k, v
            r["hbm_gbs_alg"] = round(alg / t / 1e9, 1)
            r["frac_hbm"] = round(alg / t / 1e9 / PEAK_HBM_GBS, 4)
        else:
            r["frac_mfma"] = round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        out[kind] = r
    out["varlen_lens"] = lens
    return out


def bwd_components(torch, bd, iters):
    """Training backward of the gated SWA layer at B4 S4096 (HBM-bound) and of
    a global layer at S16384 (MFMA-bound)."""
    out = {}
    for kind, tag, B, S, window, gated in (("bwd_swa_4k_b4", 6, 4, 4096, 128, True),
                                           ("bwd_global_16k", 7, 1, 16384, 0, False)):
        log(f"component: {kind}")
        l = BwdLayer(torch, bd, tag, B, S, 32, 8, window, gated)
        for _ in range(2):
            l()
        t = time_events(torch, l, iters)
        r = {"ms": round(t * 1e3, 4), "tflops": round(l.flops / t / 1e12, 2),
             "tokens_per_s": round(B * S / t, 1)}
        if window:
            r["hbm_gbs_alg"] = round(l.alg_bytes / t / 1e9, 1)
            r["frac_hbm"] = round(l.alg_bytes / t / 1e9 / PEAK_HBM_GBS, 4)
        else:
            r["frac_mfma"] = round(l.flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        out[kind] = r
        del l
        torch.cuda.empty_cache()
    return out


def decode_components(torch, bd, iters):
    """One decode step of the block's two layer kinds at 256K: B16, one new
    token at position 262144 against the global layer's 262145-key cache and
    the SWA layer's 128-slot ring."""
    from global_attention_zg_amd import inputs
    B, Hq, Hkv, L = 16, 32, 8, 262145
    out = {}
    for kind, layer, cap, ring, window, gated in (("decode_global_256k", 0, L, False, 0, False),
                                                  ("decode_swa_ring", 1, 128, True, 128, True)):
        log(f"component: {kind}")
        kc = dev_tensor(torch, (5, layer, inputs.T_KCACHE), (B, Hkv, cap, D))
        vc = dev_tensor(torch, (5, layer, inputs.T_VCACHE), (B, Hkv, cap, D))
        q = dev_tensor(torch, (5, layer, inputs.T_Q), (B, Hq, D))
        kn = dev_tensor(torch, (5, layer, inputs.T_KNEW), (B, Hkv, D))
        vn = dev_tensor(torch, (5, layer, inputs.T_VNEW), (B, Hkv, D))
        g = dev_tensor(torch, (5, layer, inputs.T_GATE), (B, Hq, D)) if gated else None
        gq = norm_w(torch, (5, layer, inputs.T_GQ))
        gk = norm_w(torch, (5, layer, inputs.T_GK))
        sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o = torch.empty_like(q)
        p = bd.make_params(B, 0, Hq, Hkv, D, window)
        ws = torch.empty(bd.zg_attn_decode_workspace_size(p, cap, 0), dtype=torch.uint8,
                         device="cuda")

        def fn():
            bd.zg_attn_decode(q, kn, vn, kc, vc, sl, ring=ring, window=window, gate=g,
                              q_norm_w=gq, k_norm_w=gk, out=o, workspace=ws, **KW)

        # the ring's 8.4 MB would stay in the caches between steps: flush
        fl = flush_buffer(torch) if ring else None

        def record(name, fn, cap, elem_bytes=2):
            for _ in range(2):
                fn()
            t, t_lo, t_hi = time_stats(torch, fn, iters, flush=fl)
            keys = min(L, cap)
            alg = B * Hkv * keys * D * 2 * elem_bytes + (q.numel() * 2 + o.numel()) * 2
            flops = B * Hq * keys * FLOP_PER_PAIR
            out[name] = {"ms": round(t * 1e3, 4), "ms_min": round(t_lo * 1e3, 4),
                         "ms_max": round(t_hi * 1e3, 4), "caches_flushed": fl is not None,
                         "tokens_per_s": round(B / t, 1),
                         "hbm_gbs_alg": round(alg / t / 1e9, 1),
                         "frac_hbm": round(alg / t / 1e9 / PEAK_HBM_GBS, 4),
                         "tflops": round(flops / t / 1e12, 3),
                         "splits": bd.zg_attn_decode_num_splits(p, cap)}

        record(kind, fn, cap)
        if not ring:
            # the same step over a paged copy of the cache: 64-token pages in
            # a scrambled order
            log(f"component: {kind}_paged")
            P = 64
            mp = (L + P - 1) // P
            gen = torch.Generator().manual_seed(5)
            bt = torch.randperm(B * mp, generator=gen).view(B, mp).to(torch.int32).cuda()
            pools = []
            for c in (kc, vc):
                pool = torch.empty((B * mp, Hkv, P, D), dtype=torch.bfloat16, device="cuda")
                full = L // P
                for b in range(B):
                    src = c[b, :, :full * P].view(Hkv, full, P, D).transpose(0, 1)
                    pool.index_copy_(0, bt[b, :full].long(), src)
                    if L % P:
                        pool[int(bt[b, full]), :, :L % P] = c[b, :, full * P:L]
                pools.append(pool)
            o_ref = o.clone()
            o_pg = torch.empty_like(o)

            def fn_paged():
                bd.zg_attn_decode_paged(q, kn, vn, pools[0], pools[1], bt, sl, window=window,
                                        gate=g, q_norm_w=gq, k_norm_w=gk, out=o_pg, workspace=ws,
                                        **KW)

            record(kind + "_paged", fn_paged, mp * P)
            out[kind + "_paged"]["page_size"] = P
            out[kind + "_paged"]["equals_contiguous"] = bool(
                torch.equal(o_pg.view(torch.int16), o_ref.view(torch.int16)))
            del pools
        # the same step over an E4M3 copy of the cache (per-tensor scales 16:
        # the N(0,1) entries then span the format's normal range)
        log(f"component: {kind}_fp8")
        kc8 = bd.zg_quantize_fp8(kc, 16.0)
        vc8 = bd.zg_quantize_fp8(vc, 16.0)
        o8 = torch.empty_like(o)

        def fn_fp8():
            bd.zg_attn_decode_fp8(q, kn, vn, kc8, vc8, sl, ring=ring, window=window,
                                  k_scale=16.0, v_scale=16.0, gate=g, q_norm_w=gq, k_norm_w=gk,
                                  out=o8, workspace=ws, **KW)

        record(kind + "_fp8", fn_fp8, cap, elem_bytes=1)
        out[kind + "_fp8"]["max_abs_vs_bf16_cache"] = round(
            float((o8.float() - o.float()).abs().max()), 5)
        del kc8, vc8
        del kc, vc, fl
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
