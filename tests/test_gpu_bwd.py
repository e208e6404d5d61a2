"""GPU parity of zg_attn_bwd (the training backward) against the fp64 oracle's
attention_bwd, through the C ABI.

The GPU side runs the forward first (its bf16 output and LSE feed the
backward, as in training); the oracle recomputes everything in fp64 from the
same bf16 inputs.  The gradient bar, per gradient tensor: relative RMS error
<= 1e-2 and max error <= 2e-2 of the tensor's largest magnitude.
"""

import sys
import zlib

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
GRADS = ("dq", "dk", "dv", "dgate", "dq_norm_w", "dk_norm_w")


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


def bwd_case(name, B, S, Hq, Hkv, gated):
    tag = 1000 + zlib.crc32(repr(name).encode()) % 100000  # stable integer seed key
    c = zc.fwd_case(tag, B, S, Hq, Hkv, gated)
    c["dout"] = zc.bits((tag, 0, inputs.T_DOUT), (B, S, Hq, zc.D))
    return c


def run_gpu(c, window, gated=True, poison=True, fwd_window=None, **kw):
    bd = _binding()
    q, k, v = (zc.to_dev(c[n], torch) for n in ("q", "k", "v"))
    g = zc.to_dev(c["gate"], torch) if gated else None
    dy = zc.to_dev(c["dout"], torch)
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    args = dict(KW)
    args.update(kw)
    out, lse = bd.zg_attn_fwd(q, k, v, g, gq, gk, want_lse=True,
                              window=window if fwd_window is None else fwd_window, **args)
    bufs = {}
    if poison:
        bufs = dict(dq=torch.full_like(q, float("nan")), dk=torch.full_like(k, float("nan")),
                    dv=torch.full_like(v, float("nan")),
                    dgate=None if g is None else torch.full_like(g, float("nan")),
                    dq_norm_w=torch.full((zc.D,), float("nan"), device="cuda"),
                    dk_norm_w=torch.full((zc.D,), float("nan"), device="cuda"))
    r = bd.zg_attn_bwd(q, k, v, g, gq, gk, out, lse, dy, window=window, **args, **bufs)
    torch.cuda.synchronize()
    res = {n: (None if r[n] is None else r[n].float().cpu().numpy().astype(np.float64))
           for n in GRADS}
    res["raw"] = r
    return res


def run_oracle(c, window, gated=True, **kw):
    args = dict(KW)
    args.update(kw)
    return orc.attention_bwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]),
                             zc.f64(c["gate"]) if gated else None, c["gq"], c["gk"],
                             zc.f64(c["dout"]), window=window, **args)


def compare_grads(got, ref, what):
    out = {}
    for n in GRADS:
        if ref[n] is None:
            assert got[n] is None
            continue
        out[n] = zc.compare_grad(got[n], ref[n], f"{what}:{n}")
    return out


@pytest.mark.parametrize("B,S,Hq,Hkv,window,gated", [
    (1, 512, 4, 1, 128, True),     # tiny pair, SWA arm
    (1, 512, 4, 1, 0, False),      # tiny pair, global arm
    (2, 300, 8, 2, 64, True),      # ragged S, two batches
    (1, 333, 8, 2, 0, False),      # ragged global
    (1, 200, 4, 4, 128, True),     # group of 1
    (1, 256, 8, 4, 0, True),       # group of 2, gated global
    (1, 160, 16, 2, 32, False),    # group of 8
    (1, 40, 4, 1, 128, True),      # S < one query block, window > S
])
def test_bwd_matches_oracle(B, S, Hq, Hkv, window, gated):
    c = bwd_case(("bwd", B, S, Hq, Hkv, window, gated), B, S, Hq, Hkv, gated)
    got = run_gpu(c, window, gated)
    ref = run_oracle(c, window, gated)
    errs = compare_grads(got, ref, f"B{B} S{S} {Hq}/{Hkv} W{window}")
    print({k: tuple(round(x, 5) for x in v) for k, v in errs.items()}, file=sys.stderr)


def test_bwd_window_at_least_s_is_global_bitwise():
    """The backward with window >= S gives the global backward's bits when
    both are fed the same forward output and LSE (the global forward's),
    up to the largest window an int holds."""
    c = bwd_case("bwd_wide", 1, 300, 8, 2, False)
    a = run_gpu(c, 0, gated=False)
    for W in (300, 301, 5000, 2 ** 31 - 1):
        b = run_gpu(c, W, gated=False, fwd_window=0)
        for n in ("dq", "dk", "dv", "dq_norm_w", "dk_norm_w"):
            assert torch.equal(a["raw"][n], b["raw"][n]), (W, n)


def test_bwd_is_deterministic():
    c = bwd_case("bwd_det", 1, 700, 8, 2, True)
    a = run_gpu(c, 128, gated=True)
    b = run_gpu(c, 128, gated=True, poison=False)
    for n in GRADS:
        assert torch.equal(a["raw"][n], b["raw"][n]), n


def test_bwd_window_one():
    """W = 1: Y = sigmoid(G) * V; dv and dG have closed forms in the oracle."""
    c = bwd_case("bwd_w1", 1, 96, 4, 1, True)
    got = run_gpu(c, 1, gated=True)
    ref = run_oracle(c, 1, gated=True)
    for n in ("dv", "dgate"):
        zc.compare_grad(got[n], ref[n], f"W1:{n}")
    # the exact dq / dk are zero; the GPU's come from bf16 rounding only
    assert np.max(np.abs(got["dq"])) < 5e-2 * np.max(np.abs(got["dv"]))
    assert np.max(np.abs(got["dk"])) < 5e-2 * np.max(np.abs(got["dv"]))


def test_bwd_single_token():
    """S = 1: the only visible key is the token itself, so P = 1 and the exact
    dq, dk and weight gradients are zero; dv and dG have closed forms."""
    c = bwd_case("bwd_s1", 2, 1, 8, 2, True)
    got = run_gpu(c, 128, gated=True)
    ref = run_oracle(c, 128, gated=True)
    for n in ("dv", "dgate"):
        zc.compare_grad(got[n], ref[n], f"S1:{n}")
    big = np.max(np.abs(got["dv"]))
    for n in ("dq", "dk", "dq_norm_w", "dk_norm_w"):
        assert np.all(np.isfinite(got[n])) and np.max(np.abs(got[n])) < 5e-2 * big, n


def test_bwd_options():
    """softmax_scale, pos_offset, rope_dim 0 and an odd rope_dim / 2."""
    c = bwd_case("bwd_opt", 1, 256, 8, 2, True)
    for kw in (dict(softmax_scale=0.05), dict(pos_offset=100000), dict(rope_dim=0),
               dict(rope_dim=30, rope_theta=1e7)):
        got = run_gpu(c, 96, gated=True, **kw)
        ref = run_oracle(c, 96, gated=True, **kw)
        compare_grads(got, ref, str(kw))


def test_bwd_swa_training_shaped_layer():
    """The SWA training layer at its real shape: B4 S4096, 32/8 heads, W 128."""
    c = bwd_case("bwd_cfg2", 4, 4096, 32, 8, True)
    got = run_gpu(c, 128, gated=True)
    ref = run_oracle(c, 128, gated=True)
    errs = compare_grads(got, ref, "cfg2")
    print(errs, file=sys.stderr)


def test_bwd_global_2k_layer():
    """A global layer at 32/8 heads, S 2048."""
    c = bwd_case("bwd_g2k", 1, 2048, 32, 8, False)
    got = run_gpu(c, 0, gated=False)
    ref = run_oracle(c, 0, gated=False)
    errs = compare_grads(got, ref, "global2k")
    print(errs, file=sys.stderr)


def test_bwd_global_16k_layer_sampled():
    """The global layer the benchmark's backward times (B1 S16384, 32/8
    heads): dq at 62 sampled rows (the first rows, tile and power-of-two
    boundaries, the last row, seeded rows) and dk, dv at 24 keys among the
    last 512 positions, against the oracle's sampled backward (which runs
    every row that sees those keys).  Every key at once through an identity:
    the rows of P sum to 1, so the sum of dV over a kv head's keys is the sum
    of dO over its group's rows and heads; that sum is held to the same bar."""
    S = 16384
    c = bwd_case("bwd_g16k", 1, S, 32, 8, False)
    got = run_gpu(c, 0, gated=False, poison=False)
    rows = inputs.global_sample_rows(S, 55, S + 1)
    rng = np.random.default_rng(S)
    keys = {S - 512, S - 300, S - 129, S - 128, S - 33, S - 32, S - 2, S - 1}
    while len(keys) < 24:
        keys.add(int(rng.integers(S - 512, S)))
    keys = sorted(keys)
    ref = orc.attention_bwd(zc.f64(c["q"]), zc.f64(c["k"]), zc.f64(c["v"]), None, c["gq"], c["gk"],
                            zc.f64(c["dout"]), window=0, rows=rows, keys=keys, **KW)
    errs = {"dq": zc.compare_grad(got["dq"][:, rows], ref["dq"], "g16k:dq"),
            "dk": zc.compare_grad(got["dk"][:, keys], ref["dk"], "g16k:dk"),
            "dv": zc.compare_grad(got["dv"][:, keys], ref["dv"], "g16k:dv")}
    dsum = zc.f64(c["dout"])[0].reshape(S, 8, 4, zc.D).sum(axis=(0, 2))   # [Hkv, D]
    errs["sum dv"] = zc.compare_grad(got["dv"][0].sum(axis=0), dsum, "g16k: sum of dv")
    print(errs, file=sys.stderr)


@pytest.mark.parametrize("rope_dim", [42, 30])
def test_bwd_q_prime_matches_oracle_prologue(rope_dim):
    """The score operand the backward uses, Q' times c = softmax scale x
    log2(e) (formed inside the dq' kernel at rope_dim 42, by the key
    prologue kernel otherwise), is the oracle's RMSNorm + partial RoPE of q,
    times c, to one bf16 rounding.  It sits at the start of the workspace
    (its first segment), rows [B,S,Hq,D]."""
    bd = _binding()
    B, S, Hq, Hkv, pos = 2, 150, 8, 2, 33
    c = bwd_case("qprime", B, S, Hq, Hkv, gated=True)
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    dy = zc.to_dev(c["dout"], torch)
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    args = dict(KW, rope_dim=rope_dim, pos_offset=pos)
    out, lse = bd.zg_attn_fwd(q, k, v, g, gq, gk, want_lse=True, window=128, **args)
    p = bd.make_params(B, S, Hq, Hkv, zc.D, 128, rope_dim, 10000.0, 1e-6, 0.0, pos)
    ws = torch.zeros(bd.zg_attn_bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    bd.zg_attn_bwd(q, k, v, g, gq, gk, out, lse, dy, window=128, workspace=ws, **args)
    torch.cuda.synchronize()
    n = B * S * Hq * zc.D
    qp = ws[:2 * n].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    qp = qp.reshape(B, S, Hq, zc.D)
    qn = orc.rms_norm(zc.f64(c["q"]), c["gq"].astype(np.float64), 1e-6)
    ref = np.stack([orc.apply_partial_rope(qn[b], pos + np.arange(S), rope_dim, 10000.0)
                    for b in range(B)])
    ref = ref * (np.log2(np.e) / np.sqrt(zc.D))
    d = np.abs(qp - ref)
    assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-5), float(d.max())
