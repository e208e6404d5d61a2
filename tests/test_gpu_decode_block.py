"""GPU parity of the single-launch block decode step (zg_attn_decode_block)
through the C ABI: every layer of a 5:1 block (five gated SWA rings and one
global layer, plus a banded linear layer in a mixed block) against the fp64
oracle's attention_decode, outputs and appended cache rows, and bit for bit
against one zg_attn_decode call per layer on copies of the same caches."""

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


def layer_case(tag, layer, B, Hq, Hkv, cap, ring, window, gated):
    key = lambda t: (tag, layer, t)  # noqa: E731
    return dict(
        q=zc.bits(key(inputs.T_Q), (B, Hq, D)),
        gate=zc.bits(key(inputs.T_GATE), (B, Hq, D)) if gated else None,
        kc=zc.bits(key(inputs.T_KCACHE), (B, Hkv, cap, D)),
        vc=zc.bits(key(inputs.T_VCACHE), (B, Hkv, cap, D)),
        kn=zc.bits(key(inputs.T_KNEW), (B, Hkv, D)),
        vn=zc.bits(key(inputs.T_VNEW), (B, Hkv, D)),
        gq=inputs.norm_weight(key(inputs.T_GQ), D),
        gk=inputs.norm_weight(key(inputs.T_GK), D),
        ring=ring, window=window, cap=cap)


def dev_layer(c):
    return dict(q=zc.to_dev(c["q"], torch), k_new=zc.to_dev(c["kn"], torch),
                v_new=zc.to_dev(c["vn"], torch), k_cache=zc.to_dev(c["kc"], torch),
                v_cache=zc.to_dev(c["vc"], torch),
                gate=None if c["gate"] is None else zc.to_dev(c["gate"], torch),
                q_norm_w=torch.from_numpy(c["gq"]).cuda(), k_norm_w=torch.from_numpy(c["gk"]).cuda(),
                ring=c["ring"], window=c["window"])


def block_5to1(tag, B, Hq, Hkv, cap_global):
    cases = [layer_case(tag, l, B, Hq, Hkv, 128, 1, 128, True) for l in range(5)]
    cases.append(layer_case(tag, 5, B, Hq, Hkv, cap_global, 0, 0, False))
    return cases


def run_block(cases, lens, workspace=None):
    bd = _binding()
    layers = [dev_layer(c) for c in cases]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for L in layers:
        L["out"] = torch.full_like(L["q"], float("nan"))
    bd.zg_attn_decode_block(layers, sl, workspace=workspace, **KW)
    torch.cuda.synchronize()
    return layers


def run_eager(cases, lens):
    """One zg_attn_decode per layer, with the block step's split counts."""
    bd = _binding()
    outs = []
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for c in cases:
        L = dev_layer(c)
        B, Hq = c["q"].shape[:2]
        p = bd.make_params(B, 0, Hq, c["kc"].shape[1], D, c["window"], **KW)
        ns = bd.zg_attn_decode_block_num_splits(p, c["cap"])
        o = bd.zg_attn_decode(L["q"], L["k_new"], L["v_new"], L["k_cache"], L["v_cache"], sl,
                              ring=c["ring"], window=c["window"], gate=L["gate"],
                              q_norm_w=L["q_norm_w"], k_norm_w=L["k_norm_w"], num_splits=ns,
                              **KW)
        outs.append((o, L["k_cache"], L["v_cache"]))
    torch.cuda.synchronize()
    return outs


def check_oracle(c, L, lens, what):
    o, _, kafter = orc.attention_decode(
        zc.f64(c["q"]), zc.f64(c["kn"]), zc.f64(c["vn"]), zc.f64(c["kc"]), zc.f64(c["vc"]), lens,
        ring=c["ring"], window=c["window"], gate=None if c["gate"] is None else zc.f64(c["gate"]),
        q_norm_w=c["gq"].astype(np.float64), k_norm_w=c["gk"].astype(np.float64), **KW)
    got = L["out"].float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), what
    zc.compare(got, o, what)
    cap = c["cap"]
    for b, n in enumerate(lens):
        slot = (n - 1) % cap if c["ring"] else min(n, cap) - 1
        gk = L["k_cache"][b, :, slot].float().cpu().numpy().astype(np.float64)
        rk = kafter[b, :, slot]
        assert np.all(np.abs(gk - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5), what
        assert torch.equal(L["v_cache"][b, :, slot].view(torch.int16).cpu(),
                           zc.to_dev(c["vn"], torch)[b].view(torch.int16).cpu()), what


def check_bitwise(layers, eager, what):
    for i, (L, (o, kc, vc)) in enumerate(zip(layers, eager)):
        assert torch.equal(L["out"].view(torch.int16), o.view(torch.int16)), f"{what} layer {i} out"
        assert torch.equal(L["k_cache"].view(torch.int16), kc.view(torch.int16)), f"{what} layer {i} k"
        assert torch.equal(L["v_cache"].view(torch.int16), vc.view(torch.int16)), f"{what} layer {i} v"


def test_block_5to1_small_parity_and_bits():
    """B6, 8/2 heads, a 1000-slot global cache: lengths on both sides of the
    ring size and of the split boundaries."""
    lens = [1, 2, 128, 129, 700, 1000]
    cases = block_5to1(601, len(lens), 8, 2, 1000)
    layers = run_block(cases, lens)
    for i, (c, L) in enumerate(zip(cases, layers)):
        check_oracle(c, L, lens, f"block layer {i}")
    check_bitwise(layers, run_eager(cases, lens), "block vs per-layer decode")


def test_block_mixed_windows_and_group_sizes():
    """A banded linear layer (window 64 over a 300-slot cache), an ungated
    global layer over the same capacity and an ungated 32-slot ring, with
    groups of 8 query heads (16/2)."""
    lens = [5, 64, 65, 300]
    cases = [layer_case(602, 0, 4, 16, 2, 300, 0, 64, True),
             layer_case(602, 1, 4, 16, 2, 300, 0, 0, False),
             layer_case(602, 2, 4, 16, 2, 32, 1, 32, False)]
    layers = run_block(cases, lens)
    for i, (c, L) in enumerate(zip(cases, layers)):
        check_oracle(c, L, lens, f"mixed layer {i}")
    check_bitwise(layers, run_eager(cases, lens), "mixed block vs per-layer decode")


def test_block_5to1_4k_two_steps_same_workspace():
    """The decode step of the 4K 5:1 block at B16, 32/8 heads, twice on one
    workspace (the split tickets return to zero after each step): the
    second step appends the next token and again matches the oracle."""
    bd = _binding()
    B = 16
    lens = [4095] * (B // 2) + [1, 17, 128, 129, 2000, 3000, 4000, 4094]
    cases = block_5to1(603, B, 32, 8, 4096)
    layers = [dev_layer(c) for c in cases]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    arr, _ = bd._block_layers(layers, sl)
    p = bd.make_params(B, 0, 32, 8, D, 0, **KW)
    ws = torch.zeros(bd.zg_attn_decode_block_workspace_size(p, arr), dtype=torch.uint8,
                     device="cuda")
    bd.zg_attn_decode_block(layers, sl, workspace=ws, **KW)
    torch.cuda.synchronize()
    for i, (c, L) in enumerate(zip(cases, layers)):
        check_oracle(c, L, lens, f"4K block step 1 layer {i}")
    # step 2: the caches now hold step 1's token; new tokens at len + 1
    lens2 = [n + 1 for n in lens]
    cases2 = []
    for c, L in zip(cases, layers):
        c2 = dict(c)
        c2["kc"] = L["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16).copy()
        c2["vc"] = L["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16).copy()
        key = (603, 100 + len(cases2), inputs.T_KNEW)
        c2["kn"] = zc.bits(key, c["kn"].shape)
        c2["vn"] = zc.bits((603, 100 + len(cases2), inputs.T_VNEW), c["vn"].shape)
        c2["q"] = zc.bits((603, 100 + len(cases2), inputs.T_Q), c["q"].shape)
        cases2.append(c2)
        L["q"] = zc.to_dev(c2["q"], torch)
        L["k_new"] = zc.to_dev(c2["kn"], torch)
        L["v_new"] = zc.to_dev(c2["vn"], torch)
        L["out"] = torch.full_like(L["q"], float("nan"))
    sl2 = torch.tensor(lens2, dtype=torch.int32, device="cuda")
    assert int(ws.view(torch.int32)[:B * 8].abs().sum().item()) == 0, "tickets not reset"
    bd.zg_attn_decode_block(layers, sl2, workspace=ws, **KW)
    torch.cuda.synchronize()
    for i, (c, L) in enumerate(zip(cases2, layers)):
        check_oracle(c, L, lens2, f"4K block step 2 layer {i}")


def test_block_argument_errors():
    bd = _binding()
    lens = [3, 4]
    cases = block_5to1(604, 2, 8, 2, 64)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    layers = [dev_layer(c) for c in cases]
    with pytest.raises(ValueError):
        bd.zg_attn_decode_block(layers + [dev_layer(cases[0])], sl, **KW)
    bad = dev_layer(cases[0])
    bad["window"] = 64  # a ring's window must equal its capacity (128)
    with pytest.raises(bd.ZgAttnError):
        bd.zg_attn_decode_block([bad], sl, **KW)
    bad = dev_layer(cases[0])
    bad["v_new"] = None  # k_new without v_new
    with pytest.raises((ValueError, bd.ZgAttnError)):
        bd.zg_attn_decode_block([bad], sl, **KW)
