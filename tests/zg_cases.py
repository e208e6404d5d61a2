"""Seeded cases and the comparison rule shared by the GPU tests, the smoke
check and the benchmark.  Inputs come from global_attention_zg_amd.inputs;
the fp64 side is widened by the oracle's own helper and the device side is a
bit-for-bit view of the same bf16 numbers."""

from __future__ import annotations

import numpy as np

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc

D = 128
# tolerance on bf16 outputs: max-abs and RMS relative to the oracle
MAX_ABS = 2e-2
REL_RMS = 1e-2


def bits(key, shape):
    return inputs.normal_bf16_bits(key, int(np.prod(shape))).reshape(shape)


def fwd_case(tag, B, S, Hq, Hkv, gated, layer=0):
    """Raw bf16 bits of q, k, v, gate and fp32 norm weights for one layer."""
    c = dict(
        q=bits((tag, layer, inputs.T_Q), (B, S, Hq, D)),
        k=bits((tag, layer, inputs.T_K), (B, S, Hkv, D)),
        v=bits((tag, layer, inputs.T_V), (B, S, Hkv, D)),
        gate=bits((tag, layer, inputs.T_GATE), (B, S, Hq, D)) if gated else None,
        gq=inputs.norm_weight((tag, layer, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, layer, inputs.T_GK), D),
    )
    return c


def to_dev(b, torch, device="cuda"):
    """uint16 bf16 bits -> a bf16 device tensor holding the same numbers."""
    if b is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(b).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def f64(b):
    return None if b is None else orc.bf16_bits_to_f64(b)


def compare(got, ref, what=""):
    """Return (max_abs, rel_rms) and assert the bf16-output tolerance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rms = float(np.sqrt(np.sum(d * d) / max(np.sum(ref * ref), 1e-300))) if d.size else 0.0
    assert max_abs <= MAX_ABS and rms <= REL_RMS, \
        f"{what}: max_abs {max_abs:.3e} (<= {MAX_ABS}), rel_rms {rms:.3e} (<= {REL_RMS})"
    return max_abs, rms


# Gradient bar of the training backward (relative, per tensor): the backward
# multiplies bf16-rounded Q', K', dO, P and dS (unit roundoff 2^-9 each) and
# accumulates in fp32, so a gradient carries a few roundoffs of relative
# error that partly cancel over the sums; measured 0.3-0.5% RMS.
GRAD_REL_RMS = 1e-2
GRAD_MAX_REL = 2e-2


def compare_grad(got, ref, what=""):
    """Return (max_err / max|ref|, rel_rms) and assert the gradient bar."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    d = got - ref
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        assert float(np.max(np.abs(got))) == 0.0, f"{what}: expected an exact zero"
        return 0.0, 0.0
    max_rel = float(np.max(np.abs(d))) / scale
    rms = float(np.sqrt(np.sum(d * d) / np.sum(ref * ref)))
    assert rms <= GRAD_REL_RMS and max_rel <= GRAD_MAX_REL, \
        f"{what}: max_err/max|ref| {max_rel:.3e} (<= {GRAD_MAX_REL}), rel_rms {rms:.3e} (<= {GRAD_REL_RMS})"
    return max_rel, rms
