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
