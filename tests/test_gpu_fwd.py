"""GPU parity of zg_attn_fwd (prologue + banded/global flash kernels) against
the fp64 oracle, through the C ABI, plus the invariants of the path."""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def _binding():
    from global_attention_zg_amd import binding
    return binding


KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)


def run_gpu(c, window, gated=True, want_lse=True, poison=True, k_out=False, **kw):
    bd = _binding()
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    g = zc.to_dev(c["gate"], torch) if gated else None
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    out = torch.empty_like(q)
    B, S, Hq, _ = q.shape
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda") if want_lse else None
    if poison:
        out.fill_(float("nan"))
        if lse is not None:
            lse.fill_(float("nan"))
    ko = torch.full_like(k, float("nan")) if k_out else None
    args = dict(KW)
    args.update(kw)
    bd.zg_attn_fwd(q, k, v, g, gq, gk, window=window, out=out, lse=lse, k_out=ko, **args)
    torch.cuda.synchronize()
    res = dict(out=out.float().cpu().numpy().astype(np.float64),
               lse=None if lse is None else lse.cpu().numpy().astype(np.float64))
    if k_out:
        res["k_out"] = ko.float().cpu().numpy().astype(np.float64)
    res["raw_out"] = out
    return res


def run_oracle(c, window, gated=True, rows=None, **kw):
    args = dict(KW)
    args.update(kw)
    return orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]),
                             zc.f64(c["gate"]) if gated else None, c["gq"].astype(np.float64),
                             c["gk"].astype(np.float64), window=window, rows=rows, **args)


def check_lse(got, ref, what):
    d = np.abs(got - ref)
    assert np.all(np.isfinite(got)), what
    assert float(d.max()) <= 2e-2, f"{what}: lse max abs {d.max():.3e}"


# --------------------------------------------------------------------------
# small and ragged shapes: full element-by-element parity
# --------------------------------------------------------------------------
@pytest.mark.parametrize("window,gated", [(128, True), (0, False), (0, True), (37, True)])
@pytest.mark.parametrize("B,S,Hq,Hkv", [(2, 1000, 8, 2), (1, 513, 4, 1)])
def test_fwd_parity_ragged(B, S, Hq, Hkv, window, gated):
    c = zc.fwd_case(101, B, S, Hq, Hkv, gated=True)
    g = run_gpu(c, window, gated)
    o, l = run_oracle(c, window, gated)
    zc.compare(g["out"], o, f"out W={window}")
    check_lse(g["lse"], l, f"lse W={window}")


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257])
@pytest.mark.parametrize("window", [128, 0])
def test_fwd_parity_odd_lengths(S, window):
    c = zc.fwd_case(102, 1, S, 8, 2, gated=True)
    g = run_gpu(c, window, gated=window > 0)
    o, l = run_oracle(c, window, gated=window > 0)
    zc.compare(g["out"], o, f"S={S} W={window}")
    check_lse(g["lse"], l, f"S={S}")


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_fwd_parity_group_sizes(grp):
    Hkv = 2
    c = zc.fwd_case(103, 1, 300, Hkv * grp, Hkv, gated=True)
    for window in (128, 0):
        g = run_gpu(c, window, gated=True)
        o, l = run_oracle(c, window, gated=True)
        zc.compare(g["out"], o, f"grp={grp} W={window}")


def test_fwd_tiny_pair_config():
    """B1 S512, 4 query / 1 KV head, W=128 gated and the global layer on the
    same inputs."""
    c = zc.fwd_case(1, 1, 512, 4, 1, gated=True)
    for window, gated in ((128, True), (0, False)):
        g = run_gpu(c, window, gated)
        o, l = run_oracle(c, window, gated)
        zc.compare(g["out"], o, f"tiny W={window}")
        check_lse(g["lse"], l, f"tiny W={window}")


@pytest.mark.parametrize("theta", [10000.0, 1e7])
def test_fwd_large_position_offset(theta):
    """Positions 262000 .. 262199, at the 10K base and at the 10M base the
    pages use for the 256K stage: outputs, LSE and the rotated keys."""
    c = zc.fwd_case(104, 1, 200, 8, 2, gated=True)
    for window in (128, 0):
        g = run_gpu(c, window, pos_offset=262000, rope_theta=theta, k_out=True)
        o, l = run_oracle(c, window, pos_offset=262000, rope_theta=theta)
        zc.compare(g["out"], o, f"pos_offset theta={theta} W={window}")
        check_lse(g["lse"], l, f"pos_offset theta={theta} W={window}")
    kn = orc.rms_norm(zc.f64(c["k"]), c["gk"].astype(np.float64), 1e-6)
    ref = orc.apply_partial_rope(kn[0], 262000 + np.arange(200), 42, theta)
    d = np.abs(g["k_out"][0] - ref)
    assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-5), float(d.max())


def test_fwd_theta_and_scale_options():
    c = zc.fwd_case(105, 1, 160, 8, 2, gated=True)
    for kw in (dict(rope_theta=1e7), dict(rope_dim=0), dict(rope_dim=64),
               dict(softmax_scale=0.05), dict(rms_eps=0.25)):
        g = run_gpu(c, 64, **kw)
        o, l = run_oracle(c, 64, **kw)
        zc.compare(g["out"], o, str(kw))
        check_lse(g["lse"], l, str(kw))


def test_k_out_is_normalised_rotated_keys():
    """The prologue's K' (returned through k_out) matches the oracle's norm +
    RoPE of the keys to bf16 rounding."""
    c = zc.fwd_case(106, 2, 150, 8, 2, gated=True)
    g = run_gpu(c, 128, k_out=True, pos_offset=77)
    kn = orc.rms_norm(zc.f64(c["k"]), c["gk"].astype(np.float64), 1e-6)
    ref = np.stack([orc.apply_partial_rope(kn[b], 77 + np.arange(150), 42, 10000.0)
                    for b in range(2)])
    d = np.abs(g["k_out"] - ref)
    assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-5), float(d.max())


# --------------------------------------------------------------------------
# invariants on the GPU path
# --------------------------------------------------------------------------
def test_gate_plus_inf_is_bitwise_ungated():
    c = zc.fwd_case(107, 1, 300, 8, 2, gated=True)
    c_inf = dict(c)
    c_inf["gate"] = np.full_like(c["gate"], 0x7F80)  # bf16 +inf
    a = run_gpu(c, 128, gated=False)["raw_out"]
    b = run_gpu(c_inf, 128, gated=True)["raw_out"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c_ninf = dict(c)
    c_ninf["gate"] = np.full_like(c["gate"], 0xFF80)  # bf16 -inf
    z = run_gpu(c_ninf, 128, gated=True)["raw_out"]
    assert torch.all(z.float() == 0)


def test_window_at_least_S_is_global():
    """The windowed kernel with window >= S computes global attention.  The
    two kernels round P to bf16 against different offsets: the windowed one
    against a running max (the row's largest weight is then exactly 1), the
    global one against a fixed bound on the row's scores.  Each weight w_j
    then carries up to 2^-9 of relative rounding in each kernel, which moves
    o = sum w_j v_j / sum w_j by at most 2^-9 max_j |v_j - o|, and each bf16
    output rounds by at most 2^-9 |o|.  So per element the two differ by at
    most 2^-8 (max|v| + 2 |o|); rel-RMS within 3e-3 and the LSE within 5e-3;
    and each meets the oracle."""
    c = zc.fwd_case(108, 2, 333, 8, 2, gated=False)
    a = run_gpu(c, 0, gated=False)
    o, l = orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), None,
                             c["gq"].astype(np.float64), c["gk"].astype(np.float64), window=0, **KW)
    zc.compare(a["out"], o, "global")
    ref = a["out"]
    vmax = float(np.abs(zc.f64(c["v"])).max())
    for W in (333, 334, 5000):
        b = run_gpu(c, W, gated=False)
        zc.compare(b["out"], o, f"W={W}")
        d = b["out"] - ref
        assert np.all(np.abs(d) <= 2.0 ** -8 * (vmax + 2 * np.abs(ref))), float(np.abs(d).max())
        assert float(np.sqrt((d * d).sum() / (ref * ref).sum())) <= 3e-3
        assert float(np.abs(b["lse"] - a["lse"]).max()) <= 5e-3


def test_window_one_is_gated_value():
    c = zc.fwd_case(109, 1, 100, 8, 2, gated=True)
    g = run_gpu(c, 1, gated=True)
    ref = orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), zc.f64(c["gate"]),
                            c["gq"].astype(np.float64), c["gk"].astype(np.float64), window=1,
                            **KW)[0]
    zc.compare(g["out"], ref, "W=1")


def test_gqa_equals_repeated_mha_on_gpu():
    c = zc.fwd_case(110, 1, 257, 8, 2, gated=True)
    c_mha = dict(c)
    c_mha["k"] = np.repeat(c["k"], 4, axis=2)
    c_mha["v"] = np.repeat(c["v"], 4, axis=2)
    for window in (128, 0):
        a = run_gpu(c, window)["out"]
        b = run_gpu(c_mha, window)["out"]
        zc.compare(a, b, f"gqa vs mha W={window}")


def test_deterministic_and_fully_written():
    c = zc.fwd_case(111, 2, 700, 8, 2, gated=True)
    for window in (128, 0):
        a = run_gpu(c, window, poison=True)
        b = run_gpu(c, window, poison=True)
        assert np.all(np.isfinite(a["out"])) and np.all(np.isfinite(a["lse"]))
        assert torch.equal(a["raw_out"].view(torch.int16), b["raw_out"].view(torch.int16))
        assert np.array_equal(a["lse"], b["lse"])


def test_without_lse_and_with_workspace_reuse():
    bd = _binding()
    c = zc.fwd_case(112, 1, 256, 8, 2, gated=True)
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    p = bd.make_params(1, 256, 8, 2, 128, 128)
    ws = torch.empty(bd.zg_attn_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    o1, l1 = bd.zg_attn_fwd(q, k, v, g, gq, gk, window=128, workspace=ws)
    assert l1 is None
    o, _ = run_oracle(c, 128)
    zc.compare(o1.float().cpu().numpy(), o, "no lse")


def test_global_forward_with_dirty_and_reused_workspace():
    """The global (causal) forward keeps its work-queue counters in the
    workspace and clears them itself: a workspace full of 0xFF bytes, the same
    workspace again right after, and a 256-byte counter-only workspace with
    k_out all give the bits of a fresh zeroed workspace."""
    bd = _binding()
    c = zc.fwd_case(114, 2, 777, 8, 2, gated=False)
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    p = bd.make_params(2, 777, 8, 2, 128, 0)
    n = bd.zg_attn_fwd_workspace_size(p)
    assert n == 2 * 777 * 2 * 128 * 2 + bd.QUEUE_BYTES
    fresh = torch.zeros(n, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = bd.zg_attn_fwd(q, k, v, None, gq, gk, window=0, want_lse=True, workspace=fresh)
    dirty = torch.full((n,), 255, dtype=torch.uint8, device="cuda")
    for rep in range(2):  # the second call finds the counters the first one left
        o, l = bd.zg_attn_fwd(q, k, v, None, gq, gk, window=0, want_lse=True, workspace=dirty)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), rep
        assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32)), rep
    ko = torch.empty_like(k)
    small = torch.full((bd.QUEUE_BYTES,), 255, dtype=torch.uint8, device="cuda")
    o, _ = bd.zg_attn_fwd(q, k, v, None, gq, gk, window=0, k_out=ko, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    ref, _ = run_oracle(c, 0, gated=False)
    zc.compare(o_ref.float().cpu().numpy(), ref, "global, dirty workspace")


def test_too_small_workspace_is_rejected_before_launch():
    bd = _binding()
    c = zc.fwd_case(113, 1, 64, 8, 2, gated=False)
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    out = torch.full_like(q, 3.0)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bd.ZgAttnError) as e:
        bd.zg_attn_fwd(q, k, v, None, gq, gk, window=0, out=out, workspace=ws)
    assert e.value.status == bd.ZG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)


@pytest.mark.parametrize("window", [256, 1000])
def test_fwd_wider_windows(window):
    """Sliding windows other than the pages' 128 (the ablation's other
    configurations): several tiles of band per query block."""
    c = zc.fwd_case(150 + window, 1, 2100, 8, 2, gated=True)
    got = run_gpu(c, window, gated=True)
    ref_out, ref_lse = run_oracle(c, window, gated=True)
    zc.compare(got["out"], ref_out, f"W{window}")
    check_lse(got["lse"], ref_lse, f"W{window}")


@pytest.mark.parametrize("window", [0, 128])
def test_fwd_large_norm_weights(window):
    """Norm weights scaled by 1.7 make the logits 2.9 times larger than
    usual: a peakier softmax, more rescaling of the running max.  The
    scores' error from rounding Q' and K' to bf16 (|ds| ~ 2^-8 |s|) grows
    with the logits, and the outputs' and the LSE's errors with it, so their
    max-abs bounds scale by 1.7^2; the rel-RMS bar stays the ordinary one."""
    c = zc.fwd_case(160 + window, 1, 700, 8, 2, gated=True)
    c["gq"] = (c["gq"] * 1.7).astype(np.float32)
    c["gk"] = (c["gk"] * 1.7).astype(np.float32)
    got = run_gpu(c, window, gated=True)
    ref_out, ref_lse = run_oracle(c, window, gated=True)
    d = got["out"] - ref_out
    assert np.all(np.isfinite(got["out"]))
    assert float(np.abs(d).max()) <= zc.MAX_ABS * 1.7 ** 2, float(np.abs(d).max())
    assert float(np.sqrt((d * d).sum() / (ref_out * ref_out).sum())) <= zc.REL_RMS
    d = np.abs(got["lse"] - ref_lse)
    assert np.all(np.isfinite(got["lse"])) and float(d.max()) <= 2e-2 * 1.7 ** 2, float(d.max())


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (8, 4), (16, 2)])
def test_global_exact_max_fallback(Hq, Hkv):
    """The global kernel offsets its softmax by a bound on each row's scores
    (|q'| sqrt(D) max|w_k|).  A key-norm weight of 8 on dimension 100 (past
    the rotary dims) where every raw key is zero makes that bound far exceed
    the row's own score, while the scores stay those of ordinary weights;
    the kernel must then take the rows' exact maxima first.  Every group
    size's wave layout goes through that path and meets the bar."""
    c = zc.fwd_case(170 + Hq + Hkv, 1, 777, Hq, Hkv, gated=False)
    k = c["k"].copy()
    k[..., 100] = 0
    c["k"] = k
    gk = c["gk"].copy()
    gk[100] = 8.0
    c["gk"] = gk
    got = run_gpu(c, 0, gated=False)
    ref_out, ref_lse = run_oracle(c, 0, gated=False)
    zc.compare(got["out"], ref_out, f"exact-max path {Hq}/{Hkv}")
    check_lse(got["lse"], ref_lse, f"exact-max path {Hq}/{Hkv}")


def test_global_long_sequence():
    """A global layer past 65536 keys (where the E4M3 variant changes its
    schedule; the bf16 kernel keeps the interleaved one at every length):
    S = 70001, 8/2 heads, sampled rows against the oracle."""
    S = 70001
    c = zc.fwd_case(180, 1, S, 8, 2, gated=False)
    g = run_gpu(c, 0, gated=False)
    rows = inputs.global_sample_rows(S, 20, S)
    o, l = run_oracle(c, 0, gated=False, rows=rows)
    zc.compare(g["out"][:, rows], o, "global S=70001")
    check_lse(g["lse"][:, :, rows], l, "global S=70001")
