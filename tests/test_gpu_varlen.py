"""GPU checks of the packed variable-length prefill (zg_attn_fwd_varlen)
through the C ABI.

Packing is a layout: sequence b's rows are computed by the same code and the
same arithmetic as zg_attn_fwd on that sequence alone, so its output, LSE
and K' rows must be bit-identical to that call; each sequence is also held
to the fp64 oracle at the bf16 output bar.
"""

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


def _binding():
    from global_attention_zg_amd import binding
    return binding


def packed_case(tag, lens, Hq, Hkv, gated):
    T = int(sum(lens))
    c = dict(
        q=zc.bits((tag, 0, inputs.T_Q), (T, Hq, D)),
        k=zc.bits((tag, 0, inputs.T_K), (T, Hkv, D)),
        v=zc.bits((tag, 0, inputs.T_V), (T, Hkv, D)),
        gate=zc.bits((tag, 0, inputs.T_GATE), (T, Hq, D)) if gated else None,
        gq=inputs.norm_weight((tag, 0, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, 0, inputs.T_GK), D),
    )
    c["cu"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return c


def _same(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def run_packed(c, window, max_seqlen, **kw):
    bd = _binding()
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    cu = torch.from_numpy(c["cu"]).cuda()
    T, Hq, _ = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    ko = torch.full_like(k, float("nan"))
    args = dict(KW)
    args.update(kw)
    bd.zg_attn_fwd_varlen(q, k, v, g, gq, gk, cu, max_seqlen, window=window, out=out, lse=lse,
                          k_out=ko, **args)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, g=g, gq=gq, gk=gk, out=out, lse=lse, ko=ko)


def run_alone(r, c, b, window, **kw):
    """zg_attn_fwd on sequence b of the packed case alone (B = 1)."""
    bd = _binding()
    s0, s1 = int(c["cu"][b]), int(c["cu"][b + 1])
    sl = lambda t: None if t is None else t[s0:s1].unsqueeze(0).contiguous()  # noqa: E731
    q, k, v, g = sl(r["q"]), sl(r["k"]), sl(r["v"]), sl(r["g"])
    ko = torch.empty_like(k)
    args = dict(KW)
    args.update(kw)
    out, lse = bd.zg_attn_fwd(q, k, v, g, r["gq"], r["gk"], window=window, want_lse=True,
                              k_out=ko, **args)
    torch.cuda.synchronize()
    return out[0], lse[0], ko[0]


def check_against_alone_and_oracle(c, r, window, oracle=True, **kw):
    for b in range(len(c["cu"]) - 1):
        s0, s1 = int(c["cu"][b]), int(c["cu"][b + 1])
        if s1 == s0:
            continue
        out, lse, ko = run_alone(r, c, b, window, **kw)
        assert _same(r["out"][s0:s1], out), f"seq {b}: out"
        assert _same(r["lse"][:, s0:s1], lse), f"seq {b}: lse"
        assert _same(r["ko"][s0:s1], ko), f"seq {b}: k_out"
        if oracle:
            args = dict(KW)
            args.update(kw)
            sl = lambda n: None if c[n] is None else zc.f64(c[n][s0:s1])[None]  # noqa: E731
            o, l = orc.attention_fwd(sl("q"), sl("k"), sl("v"), sl("gate"),
                                     c["gq"].astype(np.float64), c["gk"].astype(np.float64),
                                     window=window, **args)
            zc.compare(r["out"][s0:s1].float().cpu().numpy()[None], o, f"seq {b} vs oracle")
            d = np.abs(r["lse"][:, s0:s1].cpu().numpy()[None] - l)
            assert float(d.max()) <= 2e-2, f"seq {b}: lse max abs {d.max():.3e}"


@pytest.mark.parametrize("window,gated", [(128, True), (0, False), (64, True), (0, True)])
def test_varlen_ragged_batch(window, gated):
    lens = [300, 1, 0, 37, 513, 129, 64]
    c = packed_case(401, lens, 8, 2, gated)
    r = run_packed(c, window, max(lens))
    check_against_alone_and_oracle(c, r, window)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2), (32, 8)])
def test_varlen_group_sizes(Hq, Hkv):
    lens = [200, 65, 31]
    c = packed_case(402, lens, Hq, Hkv, True)
    r = run_packed(c, 0, max(lens))
    check_against_alone_and_oracle(c, r, 0)


def test_varlen_loose_max_seqlen_changes_nothing():
    """A grid sized for a longer sequence than any in the batch gives the
    same bits."""
    lens = [100, 250]
    c = packed_case(403, lens, 8, 2, True)
    a = run_packed(c, 0, 250)
    b = run_packed(c, 0, 4096)
    for n in ("out", "lse", "ko"):
        assert _same(a[n], b[n]), n


def test_varlen_options():
    """pos_offset, an odd rope_dim / 2 (the generic rotation path), rope 0."""
    lens = [90, 161]
    c = packed_case(404, lens, 8, 2, True)
    for kw in (dict(pos_offset=70000), dict(rope_dim=30, rope_theta=1e7), dict(rope_dim=0)):
        r = run_packed(c, 128, max(lens), **kw)
        check_against_alone_and_oracle(c, r, 128, **kw)


def test_varlen_longer_than_max_seqlen_is_cut():
    """Rows of a sequence past max_seqlen are left untouched."""
    lens = [50, 200]
    c = packed_case(405, lens, 8, 2, False)
    r = run_packed(c, 0, 120)
    assert torch.isnan(r["out"][50 + 120:]).all()
    assert not torch.isnan(r["out"][:50 + 120]).any()


def test_varlen_sixteen_sequences_of_a_mixed_serving_batch():
    """A serving-sized packed batch (16 prompts of 1..2048 tokens, 32/8
    heads, both layer kinds), bitwise equal to per-sequence calls; oracle
    on the two shortest."""
    rng = np.random.default_rng(406)
    lens = [int(x) for x in rng.integers(1, 2049, size=16)]
    c = packed_case(406, lens, 32, 8, True)
    for window in (128, 0):
        r = run_packed(c, window, max(lens))
        check_against_alone_and_oracle(c, r, window, oracle=False)
    r = run_packed(c, 0, max(lens))
    for b in np.argsort(lens)[:2]:
        s0, s1 = int(c["cu"][b]), int(c["cu"][b + 1])
        sl = lambda n: zc.f64(c[n][s0:s1])[None]  # noqa: E731
        o, _ = orc.attention_fwd(sl("q"), sl("k"), sl("v"), sl("gate"),
                                 c["gq"].astype(np.float64), c["gk"].astype(np.float64),
                                 window=0, **KW)
        zc.compare(r["out"][s0:s1].float().cpu().numpy()[None], o, f"seq {b}")
