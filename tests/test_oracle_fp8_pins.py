"""Pins of the oracle's E4M3 quantizer against the format's definition (OCP
E4M3: bias 7, 3 mantissa bits, largest finite 448, no infinities) and its
rounding rule (nearest, ties to even, saturating clamp)."""

import numpy as np

import oracle as orc


def q(v, scale=1.0):
    codes, vals = orc.quantize_e4m3(np.array([v], dtype=np.float32), scale)
    return int(codes[0]), float(vals[0])


def test_worked_values():
    assert q(1.0) == (0x38, 1.0)
    assert q(-1.0) == (0xB8, -1.0)
    assert q(0.5) == (0x30, 0.5)
    assert q(1.0625) == (0x38, 1.0)        # halfway 1 / 1.125: even mantissa 000
    assert q(1.1875) == (0x3A, 1.25)       # halfway 1.125 / 1.25: even mantissa 010
    assert q(3.14159) == (0x45, 3.25)
    assert q(-2.75) == (0xC3, -2.75)
    assert q(448.0) == (0x7E, 448.0)
    assert q(464.0) == (0x7E, 448.0)       # clamped first
    assert q(1e6) == (0x7E, 448.0)         # saturates instead of overflowing
    assert q(-1e6) == (0xFE, -448.0)
    assert q(2.0**-6) == (0x08, 2.0**-6)   # smallest normal
    assert q(2.0**-9) == (0x01, 2.0**-9)   # smallest subnormal
    assert q(2.0**-10) == (0x00, 0.0)      # halfway 0 / 2^-9: even is 0
    assert q(1.5 * 2.0**-9) == (0x02, 2.0**-8)   # halfway 2^-9 / 2^-8: even code 2
    assert q(0.003) == (0x02, 2.0**-8)
    assert q(0.25, scale=4.0) == (0x38, 1.0)     # the scale multiplies first


def test_every_finite_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3_decode(codes)
    finite = np.isfinite(vals)
    assert finite.sum() == 254 and vals[finite].max() == 448.0
    got, gv = orc.quantize_e4m3(vals[finite].astype(np.float32), 1.0)
    assert np.array_equal(got, codes[finite])
    assert np.array_equal(gv, vals[finite])


def test_rounding_error_bound_and_monotone():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))).astype(np.float32)
    codes, vals = orc.quantize_e4m3(x, 1.0)
    v = np.clip(x.astype(np.float64), -448, 448)
    a = np.abs(v)
    quantum = np.where(a < 2.0**-6, 2.0**-9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0**-6))) - 3))
    assert np.all(np.abs(vals - v) <= quantum / 2 + 1e-300)
    order = np.argsort(v)
    assert np.all(np.diff(vals[order]) >= 0)
    assert np.array_equal(orc.e4m3_decode(codes), vals)


# ---------------------------------------------------------------------------
# attention_decode_fp8: decode over an E4M3 cache, pinned by closed forms
# ---------------------------------------------------------------------------
D = 128
DEC = dict(rope_dim=0, rope_theta=10000.0, rms_eps=1e-6)


def _dec(q, kn, vn, kc, vc, lens, k_scale, v_scale, ring=False, window=0, **kw):
    args = dict(DEC)
    args.update(kw)
    ones = np.ones(D)
    return orc.attention_decode_fp8(q, kn, vn, kc, vc, lens, k_scale=k_scale, v_scale=v_scale,
                                    ring=ring, window=window, gate=None, q_norm_w=ones,
                                    k_norm_w=ones, **args)


def test_decode_fp8_uniform_scores_average_the_dequantized_values():
    """All keys zero (the appended one too: RMSNorm of 0 is 0), so every
    visible key gets weight 1/L and the output is the mean of the stored
    values, each code divided by v_scale; the new value 0.3 is stored as
    E4M3(0.3 * 4) = 1.25, i.e. 0.3125."""
    L = 5
    q = np.random.default_rng(0).standard_normal((1, 4, D))
    kc = np.zeros((1, 1, 8, D), dtype=np.uint8)
    vc = np.zeros((1, 1, 8, D), dtype=np.uint8)
    # slots 0..3: 1.0, 2.0, -1.0, 448 (codes 0x38, 0x40, 0xB8, 0x7E); slot 5 is not visible
    for s, c in enumerate((0x38, 0x40, 0xB8, 0x7E)):
        vc[0, 0, s] = c
    vc[0, 0, 5] = 0x40
    out, _, kca, vca = _dec(q, np.zeros((1, 1, D)), np.full((1, 1, D), 0.3), kc, vc, [L],
                            k_scale=2.0, v_scale=4.0)
    expect = ((1.0 + 2.0 - 1.0 + 448.0) / 4.0 + 0.3125) / L
    assert np.allclose(out, expect, rtol=1e-14, atol=0)
    assert np.all(vca[0, 0, L - 1] == 0x3A) and np.all(kca[0, 0, L - 1] == 0x00)
    assert np.array_equal(np.delete(vca, L - 1, axis=2), np.delete(vc, L - 1, axis=2))


def test_decode_fp8_two_keys_closed_form():
    """q = 5 e_0 with unit norm weights and no rotation gives
    q'_0 = 5 / sqrt(25/128 + eps) = 11.31; key 0 stores code 0x40 (= 2) in dim
    0, key 1 zeros, so the scores are tau * q'_0 * 2 / k_scale and 0 and the
    output is the two-way softmax mix of the stored values 1 / v_scale and
    -1 / v_scale.  With the query quantized: 11.31 = 0.707 * 2^4 gives the
    scale 2^(8-4) = 16, and 16 * 11.31 = 181.0 rounds to the E4M3 value 176
    (the neighbours in [128, 256) are 16 apart), so q'_0 enters as 11."""
    k_scale, v_scale = 8.0, 16.0
    q = np.zeros((1, 2, D))
    q[:, :, 0] = 5.0
    kc = np.zeros((1, 1, 4, D), dtype=np.uint8)
    kc[0, 0, 0, 0] = 0x40
    vc = np.zeros((1, 1, 4, D), dtype=np.uint8)
    vc[0, 0, 0] = 0x38
    vc[0, 0, 1] = 0xB8
    for quantize_q, qp in ((False, 5.0 / np.sqrt(25.0 / D + 1e-6)), (True, 11.0)):
        out, lse, _, _ = _dec(q, None, None, kc, vc, [2], k_scale, v_scale,
                              quantize_q=quantize_q)
        s0 = qp * 2.0 / k_scale / np.sqrt(D)
        w0 = 1.0 / (1.0 + np.exp(-s0))
        expect = (w0 - (1.0 - w0)) / v_scale
        assert np.allclose(out, expect, rtol=1e-13, atol=0), quantize_q
        assert np.allclose(lse, np.log(np.exp(s0) + 1.0), rtol=1e-13), quantize_q


def test_e4m3_row_scale_and_rows():
    """The row scale is the power of two that puts the row's amax in
    [128, 256); a row whose values are on the E4M3 grid at that scale comes
    back unchanged, and any row comes back within half an E4M3 quantum."""
    assert orc.e4m3_row_scale(np.array([[1.0, -0.5]]))[0] == 128.0     # 1 = 0.5 * 2^1
    assert orc.e4m3_row_scale(np.array([[0.75, 3.0]]))[0] == 64.0      # 3 = 0.75 * 2^2
    assert orc.e4m3_row_scale(np.array([[-448.0]]))[0] == 2.0 ** -1    # 448 = 0.875 * 2^9
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 128)) * np.exp2(rng.uniform(-8, 8, (6, 1)))
    s = orc.e4m3_row_scale(x)
    amax = np.abs(x).max(axis=1)
    assert np.all((amax * s >= 128) & (amax * s < 256))
    assert np.all(np.log2(s) == np.round(np.log2(s)))
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))       # the non-negative values
    on = rng.choice(grid[grid <= 224], (3, 128)) * rng.choice([-1, 1], (3, 128))
    on[:, 0] = 192.0                                                  # amax 192: scale 1
    assert np.array_equal(orc.e4m3_rows(on), on)
    y = orc.e4m3_rows(x)
    xs = np.abs(x * s[:, None])
    quantum = np.where(xs < 2.0**-6, 2.0**-9, np.exp2(np.floor(np.log2(np.maximum(xs, 2.0**-6))) - 3))
    assert np.all(np.abs(y - x) * s[:, None] <= quantum / 2 + 1e-300)


def test_e4m3_row_scale_clamp():
    """The exponent clamp: rows with amax >= 2^-101 keep amax * s in
    [128, 256); below that the scale stops at 2^108, which float32 still
    holds (2^108 < its largest finite value, 2^128 (1 - 2^-24)), where the
    unclamped 2^(8 - e) would overflow to inf for amax < 2^-120.  Such a row
    is then far below E4M3's smallest step (2^-9) and quantizes to zeros of
    its own signs; an all-zero row takes s = 2^8 (frexp(0) = (0, 0))."""
    f32max = float(np.finfo(np.float32).max)
    for e in (-99, -100):
        a = 0.75 * 2.0 ** e                      # = 0.75 2^e, frexp exponent e
        s = orc.e4m3_row_scale(np.array([[a, -a / 3]]))[0]
        assert s == 2.0 ** (8 - e) and 128 <= a * s < 256
    for e in (-101, -121, -140, -1074):
        a = 0.5 * 2.0 ** e if e > -1074 else 2.0 ** -1074
        s = orc.e4m3_row_scale(np.array([[a]]))[0]
        assert s == 2.0 ** 108 and s <= f32max and np.isfinite(np.float32(s))
    assert orc.e4m3_row_scale(np.zeros((1, 4)))[0] == 256.0
    tiny = np.array([[2.0 ** -123, -2.0 ** -124, 3 * 2.0 ** -125, 0.0]])
    y = orc.e4m3_rows(tiny)
    assert np.all(y == 0.0)
    assert list(np.signbit(y[0])) == [False, True, False, False]


def test_decode_fp8_ring_overwrites_the_oldest_slot():
    """Ring of 4 slots, length 6: the new token goes to slot 5 % 4 = 1,
    replacing what was there, and the 4 slots are the visible keys.  With
    zero keys the output is the mean of the 4 stored values."""
    q = np.random.default_rng(1).standard_normal((1, 1, D))
    kc = np.zeros((1, 1, 4, D), dtype=np.uint8)
    vc = np.zeros((1, 1, 4, D), dtype=np.uint8)
    for s, c in enumerate((0x38, 0x40, 0x48, 0x50)):   # 1, 2, 4, 8
        vc[0, 0, s] = c
    out, _, _, vca = _dec(q, np.zeros((1, 1, D)), np.full((1, 1, D), -0.5), kc, vc, [6],
                          k_scale=1.0, v_scale=2.0, ring=True, window=4)
    assert np.all(vca[0, 0, 1] == 0xB8)                  # -0.5 * 2 = -1
    expect = (1.0 + -1.0 + 4.0 + 8.0) / 2.0 / 4
    assert np.allclose(out, expect, rtol=1e-14, atol=0)


def test_decode_fp8_is_decode_over_the_dequantized_cache():
    """With a power-of-two scale and cache values on the E4M3 grid, the FP8
    step and the bf16-cache oracle see the same keys and values, and the new
    key is quantized from the normalised, rotated k_new."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, cap = 2, 8, 2, 40
    kc = rng.integers(0, 0x70, (B, Hkv, cap, D)).astype(np.uint8) | \
        (rng.integers(0, 2, (B, Hkv, cap, D)).astype(np.uint8) << 7)
    vc = rng.integers(0, 0x70, (B, Hkv, cap, D)).astype(np.uint8)
    q = rng.standard_normal((B, Hq, D))
    kn = rng.standard_normal((B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    gq, gk = 1.0 + 0.1 * rng.standard_normal(D), 1.0 + 0.1 * rng.standard_normal(D)
    kw = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6, pos_offset=7)
    lens = [13, 40]
    o8, l8, kca, vca = orc.attention_decode_fp8(q, kn, vn, kc, vc, lens, k_scale=64.0,
                                                v_scale=32.0, ring=False, window=0, gate=None,
                                                q_norm_w=gq, k_norm_w=gk, quantize_q=False, **kw)
    ob, lb, kafter = orc.attention_decode(q, None, None, orc.e4m3_decode(kca) / 64.0,
                                          orc.e4m3_decode(vca) / 32.0, lens, ring=False,
                                          window=0, gate=None, q_norm_w=gq, k_norm_w=gk, **kw)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
    # the appended key: the oracle's K' quantized with k_scale
    _, _, kref = orc.attention_decode(q, kn, vn, orc.e4m3_decode(kc) / 64.0,
                                      orc.e4m3_decode(vc) / 32.0, lens, ring=False, window=0,
                                      gate=None, q_norm_w=gq, k_norm_w=gk, **kw)
    for b, L in enumerate(lens):
        assert np.array_equal(kca[b, :, L - 1], orc.quantize_e4m3(kref[b, :, L - 1], 64.0)[0])
        assert np.array_equal(vca[b, :, L - 1], orc.quantize_e4m3(vn[b], 32.0)[0])


# ---------------------------------------------------------------------------
# E4M3 prefill forward (attention_fwd_fp8)
# ---------------------------------------------------------------------------
FWD = dict(rope_dim=0, rope_theta=10000.0, rms_eps=0.0)


def test_fwd_fp8_on_grid_inputs_equal_the_bf16_forward():
    """Rows of +-1 have RMS 1, so with eps 0 and no rotation q' = +-w_q and
    k' = +-w_k exactly; with weights in {0.5, 1, 1.5, 2} every q' row sits on
    the E4M3 grid at its own scale (amax 2: scale 64) and every k' on the grid
    at k_scale 16, so quantization changes nothing and the E4M3 forward is
    the plain forward."""
    rng = np.random.default_rng(21)
    B, S, Hq, Hkv = 1, 37, 4, 2
    q = rng.choice([-1.0, 1.0], (B, S, Hq, D))
    k = rng.choice([-1.0, 1.0], (B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    g = rng.standard_normal((B, S, Hq, D))
    wq = rng.choice([0.5, 1.0, 1.5, 2.0], D)
    wk = rng.choice([0.5, 1.0, 1.5, 2.0], D)
    wq[0] = wk[0] = 2.0
    for W in (0, 5):
        o8, l8 = orc.attention_fwd_fp8(q, k, v, g, wq, wk, k_scale=16.0, window=W, **FWD)
        o, l = orc.attention_fwd(q, k, v, g, wq, wk, window=W, **FWD)
        assert np.array_equal(o8, o) and np.array_equal(l8, l)


def test_fwd_fp8_two_tokens_closed_form():
    """q_0 = q_1 = k_0 = 5 e_0 and k_1 = 5 e_1, unit weights, eps 1e-6, no
    rotation: q'_0 = k'_0 = 5 / sqrt(25/128 + 1e-6) = 11.31.  The query row
    scale is 2^(8-4) = 16 and 181.0 rounds to 176, so q~'_0 = 11; at
    k_scale 3 the key gives 33.94, which rounds to 32 (the E4M3 values in
    [32, 64) are 4 apart), so k~'_0 = 32/3.  Row 0 sees only key 0 (output
    v_0, LSE s = tau 11 (32/3)); row 1 mixes v_0 (score s) and v_1 (score 0)."""
    q = np.zeros((1, 2, 1, D))
    q[..., 0] = 5.0
    k = np.zeros((1, 2, 1, D))
    k[0, 0, 0, 0] = 5.0
    k[0, 1, 0, 1] = 5.0
    v = np.random.default_rng(22).standard_normal((1, 2, 1, D))
    ones = np.ones(D)
    kw = dict(FWD, rms_eps=1e-6)
    o, lse = orc.attention_fwd_fp8(q, k, v, None, ones, ones, k_scale=3.0, window=0, **kw)
    s = 11.0 * (32.0 / 3.0) / np.sqrt(D)
    w0 = 1.0 / (1.0 + np.exp(-s))
    assert np.allclose(o[0, 0, 0], v[0, 0, 0], rtol=1e-14, atol=1e-15)
    assert np.allclose(o[0, 1, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse[0, 0], [s, np.log(np.exp(s) + 1.0)], rtol=1e-13)


def test_fwd_fp8_within_the_quantization_bound():
    """Random layer: each E4M3 value is within 2^-4 (relative) of what it
    encodes, so |s~ - s| <= tau sum_d |q'_d k'_d| (2 * 2^-4 + 2^-8) for every
    pair, and the LSE (1-Lipschitz in the max norm of a row's scores) moves
    by at most the row's largest such bound.  q' and k' for the bound come
    from the oracle's own norm and rotation."""
    rng = np.random.default_rng(23)
    B, S, Hq, Hkv = 1, 50, 4, 2
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    wq = 1 + 0.2 * rng.standard_normal(D)
    wk = 1 + 0.2 * rng.standard_normal(D)
    kw = dict(rope_dim=42, rope_theta=1e4, rms_eps=1e-6)
    _, l8 = orc.attention_fwd_fp8(q, k, v, None, wq, wk, k_scale=16.0, window=0, **kw)
    _, l = orc.attention_fwd(q, k, v, None, wq, wk, window=0, **kw)
    pos = np.arange(S)
    qp = orc.apply_partial_rope(orc.rms_norm(q[0], wq, 1e-6), pos, 42, 1e4)
    kp = orc.apply_partial_rope(orc.rms_norm(k[0], wk, 1e-6), pos, 42, 1e4)
    rel = 2 * 2.0 ** -4 + 2.0 ** -8
    for h in range(Hq):
        bound = np.abs(qp[:, h]) @ np.abs(kp[:, h // 2]).T * rel / np.sqrt(D)  # [S, S]
        bound = np.where(np.tril(np.ones((S, S), dtype=bool)), bound, 0.0).max(axis=1)
        d = np.abs(l8[0, h] - l[0, h])
        assert np.all(d <= bound + 1e-12)
        assert np.any(d > 0)      # the quantization is there
