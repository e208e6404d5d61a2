"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the training-shaped gated SWA layer (B4 S4096 32/8), the
global 16K layer, a 256K 5:1 block's SWA and global layers, and one decode
step against a 256K cache.  Where the oracle cannot finish the whole output
in seconds it is evaluated on sampled rows (or sampled (batch, kv head)
slabs for decode); every sampled row is compared element by element."""

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


def _gpu_fwd(c, window, gated):
    bd = _binding()
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    g = zc.to_dev(c["gate"], torch) if gated else None
    out = torch.full_like(q, float("nan"))
    B, S, Hq, _ = q.shape
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    bd.zg_attn_fwd(q, k, v, g, torch.from_numpy(c["gq"]).cuda(),
                   torch.from_numpy(c["gk"]).cuda(), window=window, out=out, lse=lse, **KW)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "output not fully written"
    return out, lse


def _oracle_rows(c, window, gated, rows):
    """Oracle on selected rows; for a window, only the key slice the rows need
    is handed over (positions kept through pos_offset)."""
    rows = np.asarray(sorted(rows))
    gq, gk = c["gq"].astype(np.float64), c["gk"].astype(np.float64)
    outs, lses = [], []
    if window == 0:
        s1 = int(rows.max()) + 1
        o, l = orc.attention_fwd(zc.f64(c["q"][:, :s1]), zc.f64(c["k"][:, :s1]),
                                 zc.f64(c["v"][:, :s1]),
                                 zc.f64(c["gate"][:, :s1]) if gated else None, gq, gk,
                                 window=0, rows=rows, **KW)
        return o, l
    for r in rows:
        a = max(0, int(r) - window + 1)
        sl = slice(a, int(r) + 1)
        o, l = orc.attention_fwd(zc.f64(c["q"][:, sl]), zc.f64(c["k"][:, sl]),
                                 zc.f64(c["v"][:, sl]),
                                 zc.f64(c["gate"][:, sl]) if gated else None, gq, gk,
                                 window=window, rows=[int(r) - a], pos_offset=a, **KW)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=2)


def _sample_rows(S, extra, seed):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 4095, 65535, 131071, S - 2, S - 1]
    rng = np.random.default_rng(seed)
    rows = set(r for r in fixed if 0 <= r < S)
    rows.update(int(x) for x in rng.integers(0, S, size=extra))
    return sorted(rows)


def _check_rows(out, lse, c, window, gated, rows, what):
    o_ref, l_ref = _oracle_rows(c, window, gated, rows)
    got = out[:, rows].float().cpu().numpy().astype(np.float64)
    zc.compare(got, o_ref, what)
    gl = lse[:, :, rows].cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(gl - l_ref))) <= 2e-2, what


def test_swa_training_shaped_layer_full():
    """B4 x S4096, 32/8 heads, W = 128, gated: every output element."""
    c = zc.fwd_case(2, 4, 4096, 32, 8, gated=True)
    out, lse = _gpu_fwd(c, 128, True)
    o, l = orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), zc.f64(c["gate"]),
                             c["gq"].astype(np.float64), c["gk"].astype(np.float64), window=128,
                             **KW)
    zc.compare(out.float().cpu().numpy(), o, "swa B4 S4096")
    assert float(np.max(np.abs(lse.cpu().numpy() - l))) <= 2e-2


def test_global_16k_layer_sampled_rows():
    c = zc.fwd_case(3, 1, 16384, 32, 8, gated=False)
    out, lse = _gpu_fwd(c, 0, False)
    rows = sorted(set(_sample_rows(16384, 24, 3)) | set(inputs.global_sample_rows(16384, 55, 16384)))
    _check_rows(out, lse, c, 0, False, rows, "global 16K")


def test_block_256k_swa_and_global_sampled_rows():
    """One gated SWA layer and the global layer of the 256K 5:1 block (layers
    0 and 5 of the block's independent inputs)."""
    S = 262144
    c = zc.fwd_case(4, 1, S, 32, 8, gated=True, layer=0)
    out, lse = _gpu_fwd(c, 128, True)
    _check_rows(out, lse, c, 128, True, _sample_rows(S, 16, 40), "256K swa")
    del out, lse, c
    torch.cuda.empty_cache()
    c = zc.fwd_case(4, 1, S, 32, 8, gated=False, layer=5)
    out, lse = _gpu_fwd(c, 0, False)
    # 64 rows: the first rows, tile and power-of-two boundaries, the last
    # row and seeded rows (the benchmark compares the same sample)
    _check_rows(out, lse, c, 0, False, inputs.global_sample_rows(S), "256K global")


def _fill_cache(key, B, Hkv, cap):
    """Seeded bf16 cache [B,Hkv,cap,D] built on the device one sequence at a time."""
    t = torch.empty((B, Hkv, cap, D), dtype=torch.bfloat16, device="cuda")
    per_b = Hkv * cap * D
    total = B * per_b
    for b in range(B):
        bits = inputs.normal_bf16_bits(key, total, b * per_b, (b + 1) * per_b)
        t[b] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).reshape(
            Hkv, cap, D).cuda()
    return t


def _slab(key, B, Hkv, cap, b, g):
    per = cap * D
    total = B * Hkv * per
    s0 = (b * Hkv + g) * per
    return orc.bf16_bits_to_f64(inputs.normal_bf16_bits(key, total, s0, s0 + per)).reshape(cap, D)


@pytest.mark.parametrize("layer_kind", ["global", "swa"])
def test_decode_256k_cache(layer_kind):
    """B16, one new token at position 262144 against 262144 cached positions
    (global) or the last 128 of them in a 128-slot ring (gated SWA)."""
    bd = _binding()
    B, Hq, Hkv, L = 16, 32, 8, 262145
    tag = 5
    layer = 0 if layer_kind == "global" else 1
    ring = layer_kind == "swa"
    cap = 128 if ring else L
    window = 128 if ring else 0
    kkey = (tag, layer, inputs.T_KCACHE)
    vkey = (tag, layer, inputs.T_VCACHE)
    kc = _fill_cache(kkey, B, Hkv, cap)
    vc = _fill_cache(vkey, B, Hkv, cap)
    qb = zc.bits((tag, layer, inputs.T_Q), (B, Hq, D))
    gb = zc.bits((tag, layer, inputs.T_GATE), (B, Hq, D)) if ring else None
    knb = zc.bits((tag, layer, inputs.T_KNEW), (B, Hkv, D))
    vnb = zc.bits((tag, layer, inputs.T_VNEW), (B, Hkv, D))
    gq = inputs.norm_weight((tag, layer, inputs.T_GQ), D)
    gk = inputs.norm_weight((tag, layer, inputs.T_GK), D)
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    bd.zg_attn_decode(zc.to_dev(qb, torch), zc.to_dev(knb, torch), zc.to_dev(vnb, torch), kc, vc,
                      sl, ring=ring, window=window, gate=zc.to_dev(gb, torch),
                      q_norm_w=torch.from_numpy(gq).cuda(), k_norm_w=torch.from_numpy(gk).cuda(),
                      out=out, **KW)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    grp = Hq // Hkv
    # global: one slab per sequence, the kv heads in turn (16 of 128); ring: all
    pairs = [(b, b % Hkv) for b in range(B)] if not ring else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        hs = slice(g * grp, (g + 1) * grp)
        o, _, ka = orc.decode_group(
            orc.bf16_bits_to_f64(qb[b, hs]), orc.bf16_bits_to_f64(knb[b, g]),
            orc.bf16_bits_to_f64(vnb[b, g]), _slab(kkey, B, Hkv, cap, b, g),
            _slab(vkey, B, Hkv, cap, b, g), L, ring=ring, window=window,
            gate_group=None if gb is None else orc.bf16_bits_to_f64(gb[b, hs]),
            q_norm_w=gq.astype(np.float64), k_norm_w=gk.astype(np.float64), **KW)
        zc.compare(got[b, hs], o, f"decode {layer_kind} b={b} g={g}")
        slot = (L - 1) % cap
        kw_ = kc[b, g, slot].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(kw_ - ka) <= 2.0 ** -8 * np.abs(ka) + 1e-5)
