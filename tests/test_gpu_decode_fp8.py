"""GPU parity of the E4M3-cache decode (zg_attn_decode_fp8,
zg_attn_decode_paged_fp8) against the fp64 oracle, through the C ABI.

The oracle is attention_decode_fp8: decode over the dequantized cache after
the new token's K' and V are quantized into their slot, with each query
head's row quantized to E4M3 for the QK^T product.  Outputs meet the same
bf16 bar as the bf16 cache: E4M3 products are exact in fp32 and widening a
value code to bf16 is exact, so the kernel differs from the oracle only by
fp32 summation order, the bf16 P and output, and the rare query code that
sits one step away (the kernel's fp32 q' against the oracle's fp64 q' on
either side of a rounding boundary).  Appended V codes are bit-exact (the
same fp32 product and rounding on both sides).  Appended K codes may differ
by one code step for the same reason as query codes; every other cache byte
is unchanged."""

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
K_SCALE, V_SCALE = 16.0, 32.0


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


def fp8_case(tag, B, Hq, Hkv, cap, gated=True, with_new=True):
    """bf16 inputs as for the bf16 cache; the cache is the oracle's E4M3
    codes of N(0,1) values at the test scales."""
    kv = zc.f64(zc.bits((tag, 0, inputs.T_KCACHE), (B, Hkv, cap, D)))
    vv = zc.f64(zc.bits((tag, 0, inputs.T_VCACHE), (B, Hkv, cap, D)))
    return dict(
        q=zc.bits((tag, 0, inputs.T_Q), (B, Hq, D)),
        gate=zc.bits((tag, 0, inputs.T_GATE), (B, Hq, D)) if gated else None,
        kc=orc.quantize_e4m3(kv, K_SCALE)[0],
        vc=orc.quantize_e4m3(vv, V_SCALE)[0],
        kn=zc.bits((tag, 0, inputs.T_KNEW), (B, Hkv, D)) if with_new else None,
        vn=zc.bits((tag, 0, inputs.T_VNEW), (B, Hkv, D)) if with_new else None,
        gq=inputs.norm_weight((tag, 0, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, 0, inputs.T_GK), D),
    )


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def run_gpu(c, seq_lens, ring, window, num_splits=0, **kw):
    bd = _binding()
    q = zc.to_dev(c["q"], torch)
    kc, vc = _u8(c["kc"]), _u8(c["vc"])
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    args = dict(KW)
    args.update(kw)
    bd.zg_attn_decode_fp8(q, zc.to_dev(c["kn"], torch), zc.to_dev(c["vn"], torch), kc, vc, sl,
                          ring=ring, window=window, k_scale=K_SCALE, v_scale=V_SCALE,
                          gate=zc.to_dev(c["gate"], torch),
                          q_norm_w=torch.from_numpy(c["gq"]).cuda(),
                          k_norm_w=torch.from_numpy(c["gk"]).cuda(), num_splits=num_splits,
                          out=out, **args)
    torch.cuda.synchronize()
    return out, kc, vc


def run_oracle(c, seq_lens, ring, window, **kw):
    args = dict(KW)
    args.update(kw)
    return orc.attention_decode_fp8(zc.f64(c["q"]), zc.f64(c["kn"]), zc.f64(c["vn"]), c["kc"],
                                    c["vc"], seq_lens, k_scale=K_SCALE, v_scale=V_SCALE,
                                    ring=ring, window=window, gate=zc.f64(c["gate"]),
                                    q_norm_w=c["gq"].astype(np.float64),
                                    k_norm_w=c["gk"].astype(np.float64), **args)


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_cache(kc, vc, kref, vref, slots):
    """V bit-exact everywhere; K bit-exact except at the appended slots, where
    a code may sit one step away from the oracle's (same sign, adjacent
    magnitude) on at most 1% of the elements."""
    k = kc.cpu().numpy()
    assert np.array_equal(vc.cpu().numpy(), vref)
    mask = np.zeros(k.shape, dtype=bool)
    for b, s in slots:
        mask[b, :, s] = True
    assert np.array_equal(k[~mask], kref[~mask])
    got, ref = k[mask].astype(np.int64), kref[mask].astype(np.int64)
    diff = got != ref
    if diff.any():
        assert np.all((got[diff] >> 7) == (ref[diff] >> 7))
        assert np.all(np.abs((got[diff] & 0x7F) - (ref[diff] & 0x7F)) == 1)
        assert diff.mean() <= 0.01, diff.mean()


@pytest.mark.parametrize("ring,window,cap,lens", [
    (0, 0, 1000, [1, 2, 500, 1000]),
    (1, 128, 128, [1, 50, 128, 129, 1000, 262145]),
    (0, 64, 300, [1, 63, 64, 65, 300]),
])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 16])
def test_decode_fp8_parity(ring, window, cap, lens, num_splits):
    c = fp8_case(301, len(lens), 8, 2, cap)
    out, kc, vc = run_gpu(c, lens, ring, window, num_splits=num_splits)
    o, _, kref, vref = run_oracle(c, lens, ring, window)
    zc.compare(_f(out), o, f"fp8 decode ring={ring} W={window} splits={num_splits}")
    slots = [(b, (L - 1) % cap if ring else min(L, cap) - 1) for b, L in enumerate(lens)]
    check_cache(kc, vc, kref, vref, slots)


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_decode_fp8_group_sizes(grp):
    lens = [7, 333]
    c = fp8_case(302, 2, 2 * grp, 2, 400)
    out, _, _ = run_gpu(c, lens, 0, 0)
    o, _, _, _ = run_oracle(c, lens, 0, 0)
    zc.compare(_f(out), o, f"fp8 grp={grp}")


@pytest.mark.parametrize("ring,window,cap,lens", [
    (0, 0, 300, [1, 2, 150, 300]),
    (1, 128, 128, [1, 129, 1000]),
])
def test_decode_fp8_single_split_appends_the_same_bits(ring, window, cap, lens):
    """The single-split kernel quantizes the new token itself; its cache is
    bit-identical to the separate append kernel's (several splits)."""
    c = fp8_case(303, len(lens), 8, 2, cap)
    o1, k1, v1 = run_gpu(c, lens, ring, window, num_splits=1)
    o2, k2, v2 = run_gpu(c, lens, ring, window, num_splits=2)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    o, _, _, _ = run_oracle(c, lens, ring, window)
    zc.compare(_f(o1), o, "fp8 one split")
    zc.compare(_f(o2), o, "fp8 two splits")


def test_decode_fp8_no_new_token_and_theta_options():
    """k_new = v_new = NULL (the cache already holds the token), and the
    1e7 RoPE base with a position offset."""
    lens = [40, 97, 128]
    c = fp8_case(304, 3, 8, 2, 128, with_new=False)
    for kw in (dict(), dict(rope_theta=1e7, pos_offset=100000)):
        out, kc, vc = run_gpu(c, lens, 0, 0, **kw)
        o, _, _, _ = run_oracle(c, lens, 0, 0, **kw)
        zc.compare(_f(out), o, f"fp8 no append {kw}")
        assert np.array_equal(kc.cpu().numpy(), c["kc"])
        assert np.array_equal(vc.cpu().numpy(), c["vc"])


def test_decode_fp8_tiny_query_scale_clamp():
    """Query-norm weights of 2^-125 make every head's q' row amax about
    2^-123: the row scale's exponent clamp holds the scale at 2^108 (the
    unclamped 2^131 is inf in fp32), so every query code is zero, all scores
    vanish and each head averages the visible values."""
    lens = [1, 77, 300]
    c = fp8_case(307, 3, 8, 2, 300)
    c["gq"] = np.full(D, 2.0 ** -125, dtype=np.float32)
    out, _, _ = run_gpu(c, lens, 0, 0)
    o, _, _, _ = run_oracle(c, lens, 0, 0)
    got = _f(out)
    assert np.all(np.isfinite(got))
    zc.compare(got, o, "fp8 decode tiny query")


def test_decode_fp8_every_code_widens_exactly():
    """One key takes all the weight (its stored K is 448 in every dim and
    q' = 1 in every dim, so every other score is more than 5000 below it):
    the output is that key's value row, which holds all 254 finite codes
    over two sequences.  decode(code) / v_scale is a bf16 number, so the
    output must equal it exactly."""
    bd = _binding()
    B, Hq, Hkv, cap, L, t = 2, 1, 1, 64, 64, 37
    kc = np.zeros((B, Hkv, cap, D), dtype=np.uint8)
    kc[:, :, t] = 0x7E
    vc = np.array(inputs.sign_magnitude_bytes((306, 0, inputs.T_VCACHE), B * cap * D, 0, 127),
                  dtype=np.uint8).reshape(B, Hkv, cap, D)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[np.isfinite(orc.e4m3_decode(codes))]          # 254 finite codes
    vc[0, 0, t] = codes[:128]
    vc[1, 0, t, :126] = codes[128:]
    vc[1, 0, t, 126:] = codes[:2]
    q = torch.ones((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    ones = torch.ones(D, dtype=torch.float32, device="cuda")
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    for ns in (1, 4):
        out = torch.full_like(q, float("nan"))
        bd.zg_attn_decode_fp8(q, None, None, _u8(kc), _u8(vc), sl, ring=0, window=0,
                              k_scale=1.0, v_scale=4.0, gate=None, q_norm_w=ones,
                              k_norm_w=ones, rope_dim=0, num_splits=ns, out=out)
        torch.cuda.synchronize()
        expect = orc.e4m3_decode(vc[:, 0, t]) / 4.0
        assert np.array_equal(_f(out[:, 0]), expect), ns


def test_decode_fp8_paged_bit_identical_to_contiguous():
    """Pages of 64 slots in a shuffled pool hold the same codes as the
    contiguous slabs: same output bits, same appended bytes."""
    bd = _binding()
    lens = [1, 200, 511, 64]
    B, Hq, Hkv, page = len(lens), 8, 2, 64
    max_pages = 8
    cap = max_pages * page
    c = fp8_case(305, B, Hq, Hkv, cap)
    out_c, kc, vc = run_gpu(c, lens, 0, 0, num_splits=3)
    rng = np.random.default_rng(305)
    num_pages = B * max_pages + 5
    perm = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    kp = np.zeros((num_pages, Hkv, page, D), dtype=np.uint8)
    vp = np.zeros_like(kp)
    for b in range(B):
        for j in range(max_pages):
            kp[perm[b, j]] = c["kc"][b, :, j * page:(j + 1) * page]
            vp[perm[b, j]] = c["vc"][b, :, j * page:(j + 1) * page]
    kpd, vpd = _u8(kp), _u8(vp)
    bt = torch.from_numpy(perm.astype(np.int32)).cuda()
    out_p = torch.full_like(out_c, float("nan"))
    bd.zg_attn_decode_paged_fp8(zc.to_dev(c["q"], torch), zc.to_dev(c["kn"], torch),
                                zc.to_dev(c["vn"], torch), kpd, vpd, bt,
                                torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                window=0, k_scale=K_SCALE, v_scale=V_SCALE,
                                gate=zc.to_dev(c["gate"], torch),
                                q_norm_w=torch.from_numpy(c["gq"]).cuda(),
                                k_norm_w=torch.from_numpy(c["gk"]).cuda(), num_splits=3,
                                out=out_p, **KW)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))
    kpo, vpo, kco, vco = kpd.cpu().numpy(), vpd.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()
    for b in range(B):
        for j in range(max_pages):
            assert np.array_equal(kpo[perm[b, j]], kco[b, :, j * page:(j + 1) * page])
            assert np.array_equal(vpo[perm[b, j]], vco[b, :, j * page:(j + 1) * page])


def test_decode_fp8_bad_arguments_rejected():
    bd = _binding()
    q = torch.zeros((1, 8, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 64, D), dtype=torch.uint8, device="cuda")
    sl = torch.tensor([10], dtype=torch.int32, device="cuda")
    w = torch.ones(D, dtype=torch.float32, device="cuda")
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        with pytest.raises(bd.ZgAttnError) as e:
            bd.zg_attn_decode_fp8(q, None, None, kc, kc.clone(), sl, ring=0, window=0,
                                  k_scale=ks, v_scale=vs, gate=None, q_norm_w=w, k_norm_w=w)
        assert e.value.status == bd.ZG_ERR_INVALID


def test_decode_fp8_deterministic():
    lens = [1000, 17, 512]
    c = fp8_case(307, 3, 8, 2, 1024)
    a, _, _ = run_gpu(c, lens, 0, 0, num_splits=5)
    b, _, _ = run_gpu(c, lens, 0, 0, num_splits=5)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_fp8_query_enters_quantized():
    """The two-key closed form of the oracle's pins, on the GPU: q = 5 e_0
    with unit norm weights and no rotation gives q'_0 = 11.31, which enters
    QK^T as the E4M3 value 176 / 16 = 11.  Key 0 stores 1.0 in dim 0 (k_scale
    1), key 1 zeros; values +1 and -1.  The output (2 sigma(tau * 11) - 1 =
    0.4511) is 0.011 away from what an unquantized query gives (0.4621)."""
    bd = _binding()
    q = torch.zeros((1, 1, D), dtype=torch.bfloat16, device="cuda")
    q[0, 0, 0] = 5.0
    kc = torch.zeros((1, 1, 4, D), dtype=torch.uint8, device="cuda")
    kc[0, 0, 0, 0] = 0x38
    vc = torch.zeros_like(kc)
    vc[0, 0, 0] = 0x38
    vc[0, 0, 1] = 0xB8
    ones = torch.ones(D, dtype=torch.float32, device="cuda")
    sl = torch.tensor([2], dtype=torch.int32, device="cuda")
    tau = 1.0 / np.sqrt(D)
    expect = 2.0 / (1.0 + np.exp(-tau * 11.0)) - 1.0
    unquantized = 2.0 / (1.0 + np.exp(-tau * 5.0 / np.sqrt(25.0 / D + 1e-6))) - 1.0
    for ns in (1, 2):
        out = torch.full_like(q, float("nan"))
        bd.zg_attn_decode_fp8(q, None, None, kc, vc, sl, ring=0, window=0, k_scale=1.0,
                              v_scale=1.0, gate=None, q_norm_w=ones, k_norm_w=ones, rope_dim=0,
                              num_splits=ns, out=out)
        torch.cuda.synchronize()
        got = _f(out[0, 0])
        assert np.all(np.abs(got - expect) < 2e-3), (ns, got[:4], expect)
        assert np.all(np.abs(got - unquantized) > 8e-3)


def _fill_codes(key, B, Hkv, cap, lo, hi):
    """Seeded E4M3 cache [B,Hkv,cap,D] built on the device one sequence at a
    time: magnitude codes in [lo, hi) with a random sign."""
    t = torch.empty((B, Hkv, cap, D), dtype=torch.uint8, device="cuda")
    per_b = Hkv * cap * D
    for b in range(B):
        t[b] = torch.from_numpy(inputs.sign_magnitude_bytes(key, B * per_b, lo, hi, b * per_b,
                                                            (b + 1) * per_b)).reshape(
            Hkv, cap, D).cuda()
    return t


def test_decode_fp8_256k_cache():
    """B16, one new token at position 262144 against 262144 cached positions
    in E4M3 (the bench's 256K step, automatic split count).  Codes have
    magnitudes 2^-3..15 (exponent fields 4..10), so at scale 16 the cache
    holds values in [2^-7, 0.94].  Checked against the oracle on sampled
    (sequence, KV head) groups, and the appended slot's codes."""
    bd = _binding()
    B, Hq, Hkv, L = 16, 32, 8, 262145
    tag, ks, vs = 311, 16.0, 16.0
    kkey, vkey = (tag, 0, inputs.T_KCACHE), (tag, 0, inputs.T_VCACHE)
    kc = _fill_codes(kkey, B, Hkv, L, 0x20, 0x58)
    vc = _fill_codes(vkey, B, Hkv, L, 0x20, 0x58)
    qb = zc.bits((tag, 0, inputs.T_Q), (B, Hq, D))
    knb = zc.bits((tag, 0, inputs.T_KNEW), (B, Hkv, D))
    vnb = zc.bits((tag, 0, inputs.T_VNEW), (B, Hkv, D))
    gq = inputs.norm_weight((tag, 0, inputs.T_GQ), D)
    gk = inputs.norm_weight((tag, 0, inputs.T_GK), D)
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    bd.zg_attn_decode_fp8(zc.to_dev(qb, torch), zc.to_dev(knb, torch), zc.to_dev(vnb, torch), kc,
                          vc, sl, ring=0, window=0, k_scale=ks, v_scale=vs, gate=None,
                          q_norm_w=torch.from_numpy(gq).cuda(),
                          k_norm_w=torch.from_numpy(gk).cuda(), out=out, **KW)
    torch.cuda.synchronize()
    got = _f(out)
    assert np.all(np.isfinite(got))
    grp = Hq // Hkv
    per = L * D
    for b, g in ((0, 0), (7, 3), (15, 7)):
        hs = slice(g * grp, (g + 1) * grp)
        s0 = (b * Hkv + g) * per
        kslab = inputs.sign_magnitude_bytes(kkey, B * Hkv * per, 0x20, 0x58, s0, s0 + per)
        vslab = inputs.sign_magnitude_bytes(vkey, B * Hkv * per, 0x20, 0x58, s0, s0 + per)
        o, _, kref, vref = orc.attention_decode_fp8(
            zc.f64(qb[b:b + 1, hs]), zc.f64(knb[b:b + 1, g:g + 1]), zc.f64(vnb[b:b + 1, g:g + 1]),
            kslab.reshape(1, 1, L, D), vslab.reshape(1, 1, L, D), [L], k_scale=ks, v_scale=vs,
            ring=False, window=0, gate=None, q_norm_w=gq.astype(np.float64),
            k_norm_w=gk.astype(np.float64), **KW)
        zc.compare(got[b, hs], o[0], f"fp8 decode 256K b={b} g={g}")
        assert np.array_equal(vc[b, g, L - 1].cpu().numpy(), vref[0, 0, L - 1])
        kw = kc[b, g, L - 1].cpu().numpy().astype(np.int64)
        kr = kref[0, 0, L - 1].astype(np.int64)
        assert np.all((kw == kr) | ((kw >> 7 == kr >> 7) & (np.abs((kw & 0x7F) - (kr & 0x7F)) == 1)))
