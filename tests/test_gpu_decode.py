"""GPU parity of zg_attn_decode (append, split-KV attention, LSE merge) against
the fp64 oracle, through the C ABI."""

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


def dec_case(tag, B, Hq, Hkv, cap, gated=True, with_new=True):
    return dict(
        q=zc.bits((tag, 0, inputs.T_Q), (B, Hq, D)),
        gate=zc.bits((tag, 0, inputs.T_GATE), (B, Hq, D)) if gated else None,
        kc=zc.bits((tag, 0, inputs.T_KCACHE), (B, Hkv, cap, D)),
        vc=zc.bits((tag, 0, inputs.T_VCACHE), (B, Hkv, cap, D)),
        kn=zc.bits((tag, 0, inputs.T_KNEW), (B, Hkv, D)) if with_new else None,
        vn=zc.bits((tag, 0, inputs.T_VNEW), (B, Hkv, D)) if with_new else None,
        gq=inputs.norm_weight((tag, 0, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, 0, inputs.T_GK), D),
    )


def run_gpu(c, seq_lens, ring, window, num_splits=0, **kw):
    bd = _binding()
    q = zc.to_dev(c["q"], torch)
    g = zc.to_dev(c["gate"], torch)
    kc = zc.to_dev(c["kc"], torch)
    vc = zc.to_dev(c["vc"], torch)
    kn = zc.to_dev(c["kn"], torch)
    vn = zc.to_dev(c["vn"], torch)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    args = dict(KW)
    args.update(kw)
    bd.zg_attn_decode(q, kn, vn, kc, vc, sl, ring=ring, window=window, gate=g,
                      q_norm_w=torch.from_numpy(c["gq"]).cuda(),
                      k_norm_w=torch.from_numpy(c["gk"]).cuda(), num_splits=num_splits,
                      out=out, **args)
    torch.cuda.synchronize()
    return out, kc, vc


def run_oracle(c, seq_lens, ring, window, **kw):
    args = dict(KW)
    args.update(kw)
    return orc.attention_decode(zc.f64(c["q"]), zc.f64(c["kn"]), zc.f64(c["vn"]),
                                zc.f64(c["kc"]), zc.f64(c["vc"]), seq_lens, ring=ring,
                                window=window, gate=zc.f64(c["gate"]),
                                q_norm_w=c["gq"].astype(np.float64),
                                k_norm_w=c["gk"].astype(np.float64), **args)


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("ring,window,cap,lens", [
    (0, 0, 1000, [1, 2, 500, 1000]),
    (1, 128, 128, [1, 50, 128, 129, 1000, 262145]),
    (0, 64, 300, [1, 63, 64, 65, 300]),
])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 16])
def test_decode_parity(ring, window, cap, lens, num_splits):
    c = dec_case(201, len(lens), 8, 2, cap)
    out, kc, vc = run_gpu(c, lens, ring, window, num_splits=num_splits)
    o, l, kafter = run_oracle(c, lens, ring, window)
    zc.compare(_f(out), o, f"decode ring={ring} W={window} splits={num_splits}")
    # appended cache rows: K' to bf16 rounding, V bit-exact
    for b, L in enumerate(lens):
        slot = (L - 1) % cap if ring else min(L, cap) - 1
        got = _f(kc[b, :, slot])
        ref = kafter[b, :, slot]
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
        assert torch.equal(vc[b, :, slot].view(torch.int16).cpu(),
                           zc.to_dev(c["vn"], torch)[b].view(torch.int16).cpu())


def test_decode_theta_1e7_at_256k_positions():
    """The 10M RoPE base of the 256K stage, new tokens at positions near
    262144 (pos_offset 261000 + lengths up to 1145): output and the appended
    K' rows."""
    lens = [1, 900, 1145]
    c = dec_case(206, len(lens), 8, 2, 1200)
    kw = dict(rope_theta=1e7, pos_offset=261000)
    out, kc, _ = run_gpu(c, lens, 0, 0, **kw)
    o, _, kafter = run_oracle(c, lens, 0, 0, **kw)
    zc.compare(_f(out), o, "decode theta=1e7")
    for b, L in enumerate(lens):
        got = _f(kc[b, :, L - 1])
        ref = kafter[b, :, L - 1]
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_decode_group_sizes(grp):
    lens = [7, 333]
    c = dec_case(202, 2, 2 * grp, 2, 400)
    out, _, _ = run_gpu(c, lens, 0, 0)
    o, _, _ = run_oracle(c, lens, 0, 0)
    zc.compare(_f(out), o, f"grp={grp}")


def test_decode_new_token_already_in_cache():
    """k_new = v_new = NULL: the cache already holds the new token's K', V."""
    lens = [40, 97]
    c = dec_case(203, 2, 8, 2, 128)
    out1, kc, vc = run_gpu(c, lens, 0, 0)
    bd = _binding()
    out2 = torch.full_like(out1, float("nan"))
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bd.zg_attn_decode(zc.to_dev(c["q"], torch), None, None, kc, vc, sl, ring=0, window=0,
                      gate=zc.to_dev(c["gate"], torch),
                      q_norm_w=torch.from_numpy(c["gq"]).cuda(),
                      k_norm_w=torch.from_numpy(c["gk"]).cuda(), out=out2, **KW)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("window", [0, 128])
def test_decode_equals_last_row_of_prefill(window):
    """Prefill S tokens on the GPU (k_out fills the cache), then decode the
    last token against a cache holding tokens 0..S-2: both match the oracle
    and each other."""
    bd = _binding()
    S = 300
    c = zc.fwd_case(204, 1, S, 8, 2, gated=True)
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    ko = torch.empty_like(k)
    out, _ = bd.zg_attn_fwd(q, k, v, g, gq, gk, window=window, k_out=ko, **KW)
    if window:
        cap, ring = window, 1
        kc = torch.zeros((1, 2, cap, D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        for p in range(S - 1):
            kc[0, :, p % cap] = ko[0, p]
            vc[0, :, p % cap] = v[0, p]
    else:
        cap, ring = 512, 0
        kc = torch.zeros((1, 2, cap, D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        kc[0, :, :S - 1] = ko[0, :S - 1].transpose(0, 1)
        vc[0, :, :S - 1] = v[0, :S - 1].transpose(0, 1)
    sl = torch.tensor([S], dtype=torch.int32, device="cuda")
    od = bd.zg_attn_decode(q[:, S - 1].contiguous(), k[:, S - 1].contiguous(),
                           v[:, S - 1].contiguous(), kc, vc, sl, ring=ring, window=window,
                           gate=g[:, S - 1].contiguous(), q_norm_w=gq, k_norm_w=gk, **KW)
    torch.cuda.synchronize()
    o, _ = orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), zc.f64(c["gate"]),
                             c["gq"].astype(np.float64), c["gk"].astype(np.float64),
                             window=window, rows=[S - 1], **KW)
    zc.compare(_f(od), o[:, 0], "decode vs oracle last row")
    zc.compare(_f(od), _f(out[:, S - 1]), "decode vs gpu prefill last row")


@pytest.mark.parametrize("ring,window,cap,lens", [
    (0, 0, 300, [1, 2, 150, 300]),
    (1, 128, 128, [1, 129, 1000]),
])
def test_single_split_appends_the_same_bits(ring, window, cap, lens):
    """With one split the attention kernel appends the new token itself; the
    cache it leaves is bit-identical to the one the separate append kernel
    (used with several splits) writes, and both outputs meet the bar."""
    c = dec_case(207, len(lens), 8, 2, cap)
    o1, k1, v1 = run_gpu(c, lens, ring, window, num_splits=1)
    o2, k2, v2 = run_gpu(c, lens, ring, window, num_splits=2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    o, _, _ = run_oracle(c, lens, ring, window)
    zc.compare(_f(o1), o, "one split")
    zc.compare(_f(o2), o, "two splits")


def test_decode_deterministic():
    lens = [1000, 17, 512]
    c = dec_case(205, 3, 8, 2, 1024)
    a, _, _ = run_gpu(c, lens, 0, 0, num_splits=5)
    b, _, _ = run_gpu(c, lens, 0, 0, num_splits=5)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_bad_arguments_rejected():
    bd = _binding()
    c = dec_case(206, 1, 8, 2, 64)
    q = zc.to_dev(c["q"], torch)
    kc = zc.to_dev(c["kc"], torch)
    vc = zc.to_dev(c["vc"], torch)
    sl = torch.tensor([10], dtype=torch.int32, device="cuda")
    w = torch.ones(D, dtype=torch.float32, device="cuda")
    with pytest.raises(bd.ZgAttnError) as e:   # ring requires window == cache_cap
        bd.zg_attn_decode(q, None, None, kc, vc, sl, ring=1, window=32, gate=None,
                          q_norm_w=w, k_norm_w=w)
    assert e.value.status == bd.ZG_ERR_INVALID
    with pytest.raises(bd.ZgAttnError) as e:
        bd.zg_attn_decode(q, None, None, kc, vc, sl, ring=0, window=0, gate=None, q_norm_w=w,
                          k_norm_w=w, workspace=torch.empty(16, dtype=torch.uint8,
                                                           device="cuda"))
    assert e.value.status == bd.ZG_ERR_WORKSPACE
