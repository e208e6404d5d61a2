"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws N(0,1) numbers and
rounds them to bf16, or draws uniform bytes.  Every tensor is drawn in chunks of 2**22 elements; chunk
c of tensor t for workload k, layer l comes from
``Generator(PCG64(SeedSequence([20260915, k, l, t, c])))``, so any slice can
be regenerated without materialising the whole tensor.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 20260915
CHUNK = 1 << 22

# tensor ids
T_Q, T_K, T_V, T_GATE, T_GQ, T_GK, T_KCACHE, T_VCACHE, T_KNEW, T_VNEW = range(10)
T_DOUT = 10  # upstream gradient dL/dout of the training backward
T_X, T_W = 11, 12  # layer input (hidden states) and a projection weight


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest-even bf16; return the uint16 bits."""
    u = x32.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _chunk(key, c: int, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key, c])))
    return _round_bf16_bits(g.standard_normal(n, dtype=np.float32))


def normal_bf16_bits(key, total: int, start: int = 0, stop: int | None = None,
                     out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits of elements [start, stop) of the N(0,1) tensor ``key``
    (a tuple (workload, layer, tensor)) of ``total`` elements."""
    stop = total if stop is None else stop
    assert 0 <= start <= stop <= total
    n = stop - start
    res = np.empty(n, dtype=np.uint16) if out is None else out
    c0, c1 = start // CHUNK, (stop + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        ln = min(CHUNK, total - lo)
        a = _chunk(key, c, ln)
        s0, s1 = max(start, lo), min(stop, lo + ln)
        res[s0 - start:s1 - start] = a[s0 - lo:s1 - lo]

    if c1 - c0 <= 1:
        for c in range(c0, c1):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(c0, c1)))
    return res


def scaled_normal_bf16_bits(key, total: int, scale: float) -> np.ndarray:
    """bf16 bits of N(0, scale^2) values: the float32 draws of ``key`` times
    ``scale``, rounded once to bf16 (a projection weight with fan-in n uses
    scale = n ** -0.5, so that its outputs are again of unit variance)."""
    out = np.empty(total, dtype=np.uint16)
    for c in range((total + CHUNK - 1) // CHUNK):
        lo = c * CHUNK
        ln = min(CHUNK, total - lo)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key, c])))
        out[lo:lo + ln] = _round_bf16_bits(g.standard_normal(ln, dtype=np.float32)
                                           * np.float32(scale))
    return out


def norm_weight(key, D: int) -> np.ndarray:
    """RMSNorm weight 1 + 0.1*N(0,1), rounded to a bf16-representable float32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key, 0])))
    w = (1.0 + 0.1 * g.standard_normal(D)).astype(np.float32)
    return (_round_bf16_bits(w).astype(np.uint32) << 16).view(np.float32)


def sign_magnitude_bytes(key, total: int, lo: int, hi: int, start: int = 0,
                         stop: int | None = None) -> np.ndarray:
    """Elements [start, stop) of a seeded uint8 tensor ``key`` of ``total``
    bytes: the low 7 bits uniform on [lo, hi) (0 <= lo < hi <= 128), the top
    bit a fair coin (one uniform draw x on [0, 2 (hi - lo)) per byte: the
    magnitude is lo + x // 2 and the sign x % 2).  Chunked and seeded like
    ``normal_bf16_bits``."""
    assert 0 <= lo < hi <= 128
    stop = total if stop is None else stop
    assert 0 <= start <= stop <= total
    res = np.empty(stop - start, dtype=np.uint8)

    def work(c):
        base = c * CHUNK
        ln = min(CHUNK, total - base)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key, c])))
        x = g.integers(0, 2 * (hi - lo), ln, dtype=np.uint8)
        b = (np.uint8(lo) + (x >> np.uint8(1))) | ((x & np.uint8(1)) << np.uint8(7))
        s0, s1 = max(start, base), min(stop, base + ln)
        res[s0 - start:s1 - start] = b[s0 - base:s1 - base]

    c0, c1 = start // CHUNK, (stop + CHUNK - 1) // CHUNK
    if c1 - c0 <= 1:
        for c in range(c0, c1):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(c0, c1)))
    return res


# Query rows at which a long global layer is compared with the oracle (which
# cannot afford every row of a 256K layer): the first rows, both sides of the
# first tile and 128-row boundaries, the powers of two, the last row, and
# seeded uniform rows up to 64 in all.
GLOBAL_ROWS_FIXED = (0, 1, 127, 128, 129, 4095, 65535, 131071, 262143)
GLOBAL_ROWS_SEED = 262144


def global_sample_rows(S: int = 262144, extra: int = 55, seed: int = GLOBAL_ROWS_SEED) -> list:
    rng = np.random.default_rng(seed)
    rows = set(r for r in GLOBAL_ROWS_FIXED if r < S)
    if S - 1 not in rows:
        rows.add(S - 1)
    n = min(S, len(rows) + extra)
    while len(rows) < n:
        rows.add(int(rng.integers(0, S)))
    return sorted(rows)
