"""GPU checks of the paged KV cache (zg_attn_kv_write_pages, zg_attn_decode_paged)
through the C ABI.

A paged cache is a layout, not new arithmetic: the paged decode reads the
same keys in the same order as the contiguous one, so for equal cache
contents the two outputs must agree bit for bit, and the pages written by the
append or the page fill must hold exactly the bytes of the contiguous
cache's slots.  Against the fp64 oracle the paged decode is held to the same
bf16 output bar as the contiguous decode.
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


def dec_case(tag, B, Hq, Hkv, cap, gated=True):
    return dict(
        q=zc.bits((tag, 0, inputs.T_Q), (B, Hq, D)),
        gate=zc.bits((tag, 0, inputs.T_GATE), (B, Hq, D)) if gated else None,
        kc=zc.bits((tag, 0, inputs.T_KCACHE), (B, Hkv, cap, D)),
        vc=zc.bits((tag, 0, inputs.T_VCACHE), (B, Hkv, cap, D)),
        kn=zc.bits((tag, 0, inputs.T_KNEW), (B, Hkv, D)),
        vn=zc.bits((tag, 0, inputs.T_VNEW), (B, Hkv, D)),
        gq=inputs.norm_weight((tag, 0, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, 0, inputs.T_GK), D),
    )


def page_table(seed, B, max_pages, num_pages):
    """Distinct pages in a scrambled order, drawn from a pool larger than
    needed; unused entries stay -1."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)[:B * max_pages]
    return perm.reshape(B, max_pages).astype(np.int32)


def to_pages(cache, bt, num_pages, page_size):
    """Contiguous [B,Hkv,cap,D] -> pool [num_pages,Hkv,page,D] (filler elsewhere)."""
    B, Hkv, cap, _ = cache.shape
    pool = torch.full((num_pages, Hkv, page_size, D), -7.0, dtype=cache.dtype,
                      device=cache.device)
    for b in range(B):
        for j in range(cap // page_size):
            pool[int(bt[b, j])] = cache[b, :, j * page_size:(j + 1) * page_size]
    return pool


def from_pages(pool, bt, cap):
    B = bt.shape[0]
    page_size = pool.shape[2]
    rows = [torch.cat([pool[int(bt[b, j])] for j in range(cap // page_size)], dim=1)
            for b in range(B)]
    return torch.stack(rows)


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def run_pair(c, lens, window, page_size, max_pages, num_pages, num_splits, seed):
    """The contiguous and the paged decode of one case (both append the new
    token); returns (out_contig, out_paged, cache_contig, cache_from_pages)."""
    bd = _binding()
    cap = max_pages * page_size
    q, g = zc.to_dev(c["q"], torch), zc.to_dev(c["gate"], torch)
    kn, vn = zc.to_dev(c["kn"], torch), zc.to_dev(c["vn"], torch)
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    kc, vc = zc.to_dev(c["kc"], torch), zc.to_dev(c["vc"], torch)
    B = kc.shape[0]
    bt_np = page_table(seed, B, max_pages, num_pages)
    bt = torch.from_numpy(bt_np).cuda()
    kp = to_pages(kc, bt_np, num_pages, page_size)
    vp = to_pages(vc, bt_np, num_pages, page_size)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    oc = torch.full_like(q, float("nan"))
    op = torch.full_like(q, float("nan"))
    bd.zg_attn_decode(q, kn, vn, kc, vc, sl, ring=0, window=window, gate=g, q_norm_w=gq,
                      k_norm_w=gk, num_splits=num_splits, out=oc, **KW)
    bd.zg_attn_decode_paged(q, kn, vn, kp, vp, bt, sl, window=window, gate=g, q_norm_w=gq,
                            k_norm_w=gk, num_splits=num_splits, out=op, **KW)
    torch.cuda.synchronize()
    return oc, op, (kc, vc), (from_pages(kp, bt_np, cap), from_pages(vp, bt_np, cap))


@pytest.mark.parametrize("page_size,max_pages,window,lens", [
    (32, 10, 0, [1, 31, 32, 33, 320]),        # smallest page; lens at page edges
    (64, 6, 64, [1, 63, 65, 200, 384]),       # windowed read straddling pages
    (256, 4, 0, [255, 256, 257, 1024]),
    (1024, 2, 0, [1, 2048]),
])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_paged_equals_contiguous_bitwise(page_size, max_pages, window, lens, num_splits):
    cap = page_size * max_pages
    c = dec_case(301, len(lens), 8, 2, cap)
    oc, op, (kc, vc), (kq, vq) = run_pair(c, lens, window, page_size, max_pages,
                                          num_pages=len(lens) * max_pages + 3,
                                          num_splits=num_splits, seed=page_size + num_splits)
    assert _same(oc, op)
    # the append wrote the same bytes into the page slot as into the slab
    assert _same(kc, kq) and _same(vc, vq)
    o, _, _ = orc.attention_decode(zc.f64(c["q"]), zc.f64(c["kn"]), zc.f64(c["vn"]),
                                   zc.f64(c["kc"]), zc.f64(c["vc"]), lens, ring=0,
                                   window=window, gate=zc.f64(c["gate"]),
                                   q_norm_w=c["gq"].astype(np.float64),
                                   k_norm_w=c["gk"].astype(np.float64), **KW)
    zc.compare(_f(op), o, f"paged P{page_size} W{window} splits={num_splits}")


@pytest.mark.parametrize("grp", [1, 4, 8])
def test_paged_group_sizes(grp):
    lens = [77, 130]
    c = dec_case(302, 2, 2 * grp, 2, 192)
    oc, op, _, _ = run_pair(c, lens, 0, 64, 3, num_pages=9, num_splits=0, seed=grp)
    assert _same(oc, op)


def test_write_pages_then_decode_matches_prefill():
    """Prefill S tokens (k_out = K'), fill a page pool from K' and V, decode
    token S-1 against the pool without appending: equals the prefill's last
    row (to the bar) and the oracle."""
    bd = _binding()
    B, S, Hq, Hkv, P, max_pages = 2, 300, 8, 2, 64, 6
    c = zc.fwd_case(303, B, S, Hq, Hkv, gated=True)
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    ko = torch.empty_like(k)
    out, _ = bd.zg_attn_fwd(q, k, v, g, gq, gk, window=0, k_out=ko, **KW)
    num_pages = 17
    bt_np = page_table(7, B, max_pages, num_pages)
    bt = torch.from_numpy(bt_np).cuda()
    kp = torch.full((num_pages, Hkv, P, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    bd.zg_attn_kv_write_pages(ko, v, kp, vp, bt)
    torch.cuda.synchronize()
    # every written slot holds the exact bytes of K' / V
    kq = from_pages(kp, bt_np, max_pages * P)[:, :, :S]
    vq = from_pages(vp, bt_np, max_pages * P)[:, :, :S]
    assert _same(kq, ko.transpose(1, 2).contiguous())
    assert _same(vq, v.transpose(1, 2).contiguous())
    sl = torch.tensor([S, S], dtype=torch.int32, device="cuda")
    od = bd.zg_attn_decode_paged(q[:, S - 1].contiguous(), None, None, kp, vp, bt, sl, window=0,
                                 gate=g[:, S - 1].contiguous(), q_norm_w=gq, k_norm_w=gk, **KW)
    torch.cuda.synchronize()
    o, _ = orc.attention_fwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), zc.f64(c["gate"]),
                             c["gq"].astype(np.float64), c["gk"].astype(np.float64),
                             window=0, rows=[S - 1], **KW)
    zc.compare(_f(od), o[:, 0], "paged decode vs oracle last row")
    zc.compare(_f(od), _f(out[:, S - 1]), "paged decode vs gpu prefill last row")


def test_write_pages_ragged_tail_leaves_other_slots():
    """S not a multiple of the page size: slots past S and pages outside the
    table keep their contents."""
    bd = _binding()
    B, S, Hkv, P = 1, 70, 2, 32
    k = zc.to_dev(zc.bits((304, 0, inputs.T_K), (B, S, Hkv, D)), torch)
    v = zc.to_dev(zc.bits((304, 0, inputs.T_V), (B, S, Hkv, D)), torch)
    kp = torch.full((5, Hkv, P, D), 3.0, dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, 3.0)
    bt_np = np.array([[4, 0, 2]], dtype=np.int32)
    bd.zg_attn_kv_write_pages(k, v, kp, vp, torch.from_numpy(bt_np).cuda())
    torch.cuda.synchronize()
    got = from_pages(kp, bt_np, 3 * P)
    assert _same(got[:, :, :S], k.transpose(1, 2).contiguous())
    assert torch.all(got[:, :, S:] == 3.0)
    assert torch.all(kp[1] == 3.0) and torch.all(kp[3] == 3.0)
    assert torch.all(vp[1] == 3.0) and torch.all(vp[3] == 3.0)


def test_shared_prefix_pages():
    """Two sequences whose tables share their first pages (a common prompt)
    read them without copies; each output equals the contiguous decode of a
    cache holding the shared prefix."""
    bd = _binding()
    P, max_pages, Hq, Hkv = 64, 4, 8, 2
    cap = P * max_pages
    c = dec_case(305, 2, Hq, Hkv, cap)
    kc, vc = zc.to_dev(c["kc"], torch), zc.to_dev(c["vc"], torch)
    kc[1, :, :2 * P] = kc[0, :, :2 * P]  # sequence 1 starts with sequence 0's two pages
    vc[1, :, :2 * P] = vc[0, :, :2 * P]
    bt_np = np.array([[3, 5, 0, 1], [3, 5, 6, 2]], dtype=np.int32)
    kp = torch.zeros((7, Hkv, P, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    for b in range(2):
        for j in range(max_pages):
            kp[int(bt_np[b, j])] = kc[b, :, j * P:(j + 1) * P]
            vp[int(bt_np[b, j])] = vc[b, :, j * P:(j + 1) * P]
    q, g = zc.to_dev(c["q"], torch), zc.to_dev(c["gate"], torch)
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    sl = torch.tensor([150, 200], dtype=torch.int32, device="cuda")
    oc = bd.zg_attn_decode(q, None, None, kc, vc, sl, ring=0, window=0, gate=g, q_norm_w=gq,
                           k_norm_w=gk, **KW)
    op = bd.zg_attn_decode_paged(q, None, None, kp, vp, torch.from_numpy(bt_np).cuda(), sl,
                                 window=0, gate=g, q_norm_w=gq, k_norm_w=gk, **KW)
    torch.cuda.synchronize()
    assert _same(oc, op)


def test_unused_table_entries_are_not_read():
    """Entries past a sequence's last page may be anything (here -1 and a
    huge id); the output is that of the valid pages alone."""
    bd = _binding()
    P, max_pages = 32, 8
    lens = [40, 64]  # two pages each
    c = dec_case(306, 2, 8, 2, P * max_pages)
    bt_np = np.full((2, max_pages), -1, dtype=np.int32)
    bt_np[0, :2] = [2, 0]
    bt_np[1, :2] = [1, 3]
    bt_np[1, 2:] = 1 << 30
    kc, vc = zc.to_dev(c["kc"], torch), zc.to_dev(c["vc"], torch)
    kp = torch.zeros((4, 2, P, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    for b in range(2):
        for j in range(2):
            kp[int(bt_np[b, j])] = kc[b, :, j * P:(j + 1) * P]
            vp[int(bt_np[b, j])] = vc[b, :, j * P:(j + 1) * P]
    q, g = zc.to_dev(c["q"], torch), zc.to_dev(c["gate"], torch)
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    oc = bd.zg_attn_decode(q, None, None, kc, vc, sl, ring=0, window=0, gate=g, q_norm_w=gq,
                           k_norm_w=gk, **KW)
    op = bd.zg_attn_decode_paged(q, None, None, kp, vp, torch.from_numpy(bt_np).cuda(), sl,
                                 window=0, gate=g, q_norm_w=gq, k_norm_w=gk, **KW)
    torch.cuda.synchronize()
    assert _same(oc, op)


def test_paged_deterministic_and_rejects_bad_page_size():
    bd = _binding()
    lens = [500, 3]
    c = dec_case(307, 2, 8, 2, 512)
    _, a, _, _ = run_pair(c, lens, 0, 128, 4, num_pages=9, num_splits=5, seed=1)
    _, b, _, _ = run_pair(c, lens, 0, 128, 4, num_pages=9, num_splits=5, seed=2)
    assert _same(a, b)
    q = zc.to_dev(c["q"], torch)
    pool = torch.zeros((4, 2, 48, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    with pytest.raises(bd.ZgAttnError):
        bd.zg_attn_decode_paged(q, None, None, pool, pool, bt, sl, window=0, gate=None,
                                q_norm_w=torch.ones(D, device="cuda"),
                                k_norm_w=torch.ones(D, device="cuda"), **KW)
