"""GPU parity of the E4M3 prefill forward (zg_attn_fwd_fp8) against the fp64
oracle's attention_fwd_fp8, through the C ABI.

The kernel and the oracle quantize the same numbers: K' * k_scale (per
tensor) and each query head's row q' (its own power-of-two scale).  E4M3
products are exact and the sums are fp32, so the outputs meet the bf16 bar
of the other forward tests; what differs is the fp32 summation order, P
rounded to bf16, and the rare code that sits one E4M3 step away (the
kernel's fp32 K' or q' against the oracle's fp64 value on either side of a
rounding boundary).  The K' codes the kernel writes are compared code by
code on that rule: the same code, or the neighbouring one of the same sign
on at most 1% of the elements."""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
D = 128


@pytest.fixture(autouse=True)
def _gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _binding():
    from global_attention_zg_amd import binding
    return binding


def run_gpu(c, k_scale, gated=False, window=0, **kw):
    bd = _binding()
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    g = zc.to_dev(c["gate"], torch) if gated else None
    B, S, Hq, _ = q.shape
    Hkv = k.shape[2]
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    codes = torch.zeros((B, S, Hkv, D), dtype=torch.uint8, device="cuda")
    args = dict(KW)
    args.update(kw)
    bd.zg_attn_fwd_fp8(q, k, v, g, torch.from_numpy(c["gq"]).cuda(),
                       torch.from_numpy(c["gk"]).cuda(), k_scale=k_scale, window=window, out=out,
                       lse=lse, k_out=codes, **args)
    torch.cuda.synchronize()
    return dict(out=out.float().cpu().numpy().astype(np.float64),
                lse=lse.cpu().numpy().astype(np.float64), codes=codes.cpu().numpy(), raw=out)


def run_oracle(c, k_scale, gated=False, rows=None, **kw):
    args = dict(KW)
    args.update(kw)
    return orc.attention_fwd_fp8(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]),
                                 zc.f64(c["gate"]) if gated else None,
                                 c["gq"].astype(np.float64), c["gk"].astype(np.float64),
                                 k_scale=k_scale, window=0, rows=rows, **args)


def oracle_codes(c, k_scale, pos_offset=0, rope_dim=42, rope_theta=10000.0):
    kn = orc.rms_norm(zc.f64(c["k"]), c["gk"].astype(np.float64), 1e-6)
    S = kn.shape[1]
    kp = np.stack([orc.apply_partial_rope(kn[b], pos_offset + np.arange(S), rope_dim, rope_theta)
                   for b in range(kn.shape[0])])
    return orc.quantize_e4m3(kp, k_scale)[0]


def check_codes(got, ref):
    diff = got != ref
    if diff.any():
        g, r = got[diff].astype(np.int64), ref[diff].astype(np.int64)
        assert np.all((g >> 7) == (r >> 7))
        assert np.all(np.abs((g & 0x7F) - (r & 0x7F)) == 1)
        assert diff.mean() <= 0.01, diff.mean()


def check_lse(got, ref, what):
    d = np.abs(got - ref)
    assert np.all(np.isfinite(got)), what
    assert float(d.max()) <= 2e-2, f"{what}: lse max abs {d.max():.3e}"


@pytest.mark.parametrize("k_scale", [16.0, 3.0])
@pytest.mark.parametrize("B,S,Hq,Hkv,gated", [(2, 1000, 8, 2, False), (1, 513, 4, 1, True),
                                               (1, 300, 16, 2, False)])
def test_fwd_fp8_parity(B, S, Hq, Hkv, gated, k_scale):
    c = zc.fwd_case(401, B, S, Hq, Hkv, gated=True)
    g = run_gpu(c, k_scale, gated)
    o, l = run_oracle(c, k_scale, gated)
    zc.compare(g["out"], o, f"fp8 B{B} S{S} {Hq}/{Hkv} k_scale={k_scale}")
    check_lse(g["lse"], l, "fp8")
    check_codes(g["codes"], oracle_codes(c, k_scale))


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257])
def test_fwd_fp8_odd_lengths(S):
    c = zc.fwd_case(402, 1, S, 8, 2, gated=False)
    g = run_gpu(c, 16.0)
    o, l = run_oracle(c, 16.0)
    zc.compare(g["out"], o, f"fp8 S={S}")
    check_lse(g["lse"], l, f"fp8 S={S}")


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_fwd_fp8_group_sizes(grp):
    c = zc.fwd_case(403, 1, 300, 2 * grp, 2, gated=False)
    g = run_gpu(c, 8.0)
    o, _ = run_oracle(c, 8.0)
    zc.compare(g["out"], o, f"fp8 grp={grp}")


def test_fwd_fp8_options():
    """Other rotary widths (register and LDS rotation paths), the 10M base at
    positions near 262144, an explicit softmax scale."""
    c = zc.fwd_case(404, 1, 200, 8, 2, gated=False)
    for kw in (dict(rope_dim=0), dict(rope_dim=30), dict(rope_theta=1e7, pos_offset=262000),
               dict(softmax_scale=0.05)):
        g = run_gpu(c, 16.0, **kw)
        o, l = run_oracle(c, 16.0, **kw)
        zc.compare(g["out"], o, str(kw))
        check_lse(g["lse"], l, str(kw))
        ok = {k: kw[k] for k in ("pos_offset", "rope_dim", "rope_theta") if k in kw}
        check_codes(g["codes"], oracle_codes(c, 16.0, **ok))


def test_fwd_fp8_window_at_least_s_is_global_and_band_rejected():
    bd = _binding()
    c = zc.fwd_case(405, 1, 100, 8, 2, gated=False)
    a = run_gpu(c, 16.0)["raw"]
    b = run_gpu(c, 16.0, window=100)["raw"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(bd.ZgAttnError):
        run_gpu(c, 16.0, window=99)
    with pytest.raises(bd.ZgAttnError):
        run_gpu(c, 0.0)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 8)])
def test_fwd_fp8_exact_max_fallback(Hq, Hkv):
    """As for the bf16 kernel: a key-norm weight of 8 on a dimension where
    every raw key is zero makes the score bound far exceed each row's own
    score, so the kernel takes the exact row maxima first (k_scale 4 keeps
    K' * k_scale inside the E4M3 range)."""
    c = zc.fwd_case(406 + Hkv, 1, 700, Hq, Hkv, gated=False)
    k = c["k"].copy()
    k[..., 100] = 0
    c["k"] = k
    gk = c["gk"].copy()
    gk[100] = 8.0
    c["gk"] = gk
    g = run_gpu(c, 4.0)
    o, l = run_oracle(c, 4.0)
    zc.compare(g["out"], o, f"fp8 exact-max {Hq}/{Hkv}")
    check_lse(g["lse"], l, "fp8 exact-max")


def test_fwd_fp8_deterministic():
    c = zc.fwd_case(407, 1, 1000, 8, 2, gated=False)
    a = run_gpu(c, 16.0)["raw"]
    b = run_gpu(c, 16.0)["raw"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fwd_fp8_global_16k_sampled_rows():
    """The global layer at B1 S16384, 32/8 heads (the bf16 16K workload's
    shape): the 62-row sample against the oracle, all 32 heads."""
    S = 16384
    c = zc.fwd_case(408, 1, S, 32, 8, gated=False)
    g = run_gpu(c, 16.0)
    rows = inputs.global_sample_rows(S, 55, S)
    o, l = run_oracle(c, 16.0, rows=rows)
    zc.compare(g["out"][:, rows], o, "fp8 global 16K")
    check_lse(g["lse"][:, :, rows], l, "fp8 global 16K")
    check_codes(g["codes"], oracle_codes(c, 16.0))


def test_fwd_fp8_long_sequence_schedule():
    """The E4M3 kernel past 65536 keys (the non-interleaved schedule):
    S = 70001, 8/2 heads, sampled rows against the oracle."""
    S = 70001
    c = zc.fwd_case(409, 1, S, 8, 2, gated=False)
    g = run_gpu(c, 16.0)
    rows = inputs.global_sample_rows(S, 20, S)
    o, l = run_oracle(c, 16.0, rows=rows)
    zc.compare(g["out"][:, rows], o, "fp8 global S=70001")
    check_lse(g["lse"][:, :, rows], l, "fp8 global S=70001")
