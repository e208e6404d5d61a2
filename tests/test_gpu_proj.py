"""GPU parity of the projection GEMMs (zg_linear, zg_qkvg_proj) against the
oracle's fp64 linear maps, through the C ABI.

Inputs are N(0,1) hidden states and weights of variance 1 / fan-in, both
bf16, so every output is of unit scale: the bf16 output bar (max-abs 2e-2,
rel-RMS 1e-2) applies as it does to attention.  The GPU accumulates in fp32
over K terms (error ~ sqrt(K) 2^-24 relative) and rounds once to bf16
(2^-9 relative).
"""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

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


def xw(tag, M, N, K):
    x = zc.bits((tag, 0, inputs.T_X), (M, K))
    w = inputs.scaled_normal_bf16_bits((tag, 0, inputs.T_W), N * K, K ** -0.5).reshape(N, K)
    return x, w


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [
    (1, 256, 32),        # one row, one tile, one K step
    (100, 512, 64),      # ragged M inside one tile
    (257, 256, 96),      # one row past a tile; K not a multiple of the ring
    (1000, 1024, 4096),  # several tiles, the model's K
    (2048, 4096, 4096),  # the output projection of 2048 tokens
])
def test_linear_matches_oracle(M, N, K):
    bd = _binding()
    x, w = xw(600 + M, M, N, K)
    y = bd.zg_linear(zc.to_dev(x, torch), zc.to_dev(w, torch))
    torch.cuda.synchronize()
    ref = orc.linear(zc.f64(x), zc.f64(w))
    zc.compare(_f(y), ref, f"linear {M}x{N}x{K}")


def test_linear_writes_only_its_rows_and_is_deterministic():
    bd = _binding()
    M, N, K = 300, 512, 128
    x, w = xw(610, M, N, K)
    xd, wd = zc.to_dev(x, torch), zc.to_dev(w, torch)
    big = torch.full((M + 64, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    bd.zg_linear(xd, wd, out=big[:M])
    y2 = bd.zg_linear(xd, wd)
    torch.cuda.synchronize()
    assert torch.isnan(big[M:]).all()
    assert torch.equal(big[:M].view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("Hq,Hkv,gated", [(32, 8, True), (32, 8, False), (8, 2, True)])
def test_qkvg_proj_matches_oracle(Hq, Hkv, gated):
    bd = _binding()
    T, hidden = 300, 4096 if Hq == 32 else 512
    N = 2 * Hkv * D + (2 if gated else 1) * Hq * D
    x, w = xw(620 + Hq + int(gated), T, N, hidden)
    q, k, v, g = bd.zg_qkvg_proj(zc.to_dev(x, torch), zc.to_dev(w, torch), Hq, Hkv, gated)
    torch.cuda.synchronize()
    rq, rk, rv, rg = orc.qkvg_proj(zc.f64(x), zc.f64(w), Hq, Hkv, D, gated)
    zc.compare(_f(q), rq, "q")
    zc.compare(_f(k), rk, "k")
    zc.compare(_f(v), rv, "v")
    if gated:
        zc.compare(_f(g), rg, "gate")
    else:
        assert g is None


def test_projection_feeds_attention():
    """x -> zg_qkvg_proj -> zg_attn_fwd (gated SWA layer) against the oracle
    chain qkvg_proj -> attention_fwd in fp64; the GPU rounds q, k, v and the
    gate to bf16 in between."""
    bd = _binding()
    T, hidden, Hq, Hkv = 200, 512, 8, 2
    N = 2 * Hkv * D + 2 * Hq * D
    x, w = xw(630, T, N, hidden)
    gq = inputs.norm_weight((630, 0, inputs.T_GQ), D)
    gk = inputs.norm_weight((630, 0, inputs.T_GK), D)
    q, k, v, g = bd.zg_qkvg_proj(zc.to_dev(x, torch), zc.to_dev(w, torch), Hq, Hkv, True)
    kw = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
    out, _ = bd.zg_attn_fwd(q[None], k[None], v[None], g[None], torch.from_numpy(gq).cuda(),
                            torch.from_numpy(gk).cuda(), window=128, **kw)
    torch.cuda.synchronize()
    rq, rk, rv, rg = orc.qkvg_proj(zc.f64(x), zc.f64(w), Hq, Hkv, D, True)
    ro, _ = orc.attention_fwd(rq[None], rk[None], rv[None], rg[None], gq.astype(np.float64),
                              gk.astype(np.float64), window=128, **kw)
    zc.compare(_f(out), ro, "projection -> attention")


def test_full_size_input_projection_sampled_rows():
    """The gated layer's input projection at 4096 tokens (10240 x 4096
    weight); the oracle checks 48 sampled token rows."""
    bd = _binding()
    T, hidden, Hq, Hkv = 4096, 4096, 32, 8
    N = 2 * Hkv * D + 2 * Hq * D
    x, w = xw(640, T, N, hidden)
    q, k, v, g = bd.zg_qkvg_proj(zc.to_dev(x, torch), zc.to_dev(w, torch), Hq, Hkv, True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(640).choice(T, 48, replace=False))
    rows[0], rows[-1] = 0, T - 1
    y = np.concatenate([_f(t).reshape(T, -1)[rows] for t in (q, k, v, g)], axis=1)
    ref = orc.linear(zc.f64(x[rows]), zc.f64(w))
    zc.compare(y, ref, "sampled rows")
