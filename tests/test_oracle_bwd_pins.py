"""Pins of the oracle's backward (attention_bwd, rope_bwd, rms_norm_bwd).

The backward is the derivative of the forward, so its strongest pin is the
forward itself: central finite differences of L = sum(dY * Y(theta)) through
the (separately pinned) forward oracle, entry by entry, for every input that
has a gradient.  Closed forms and special cases pin the rest:

* window 1: Y = sigmoid(G) * V_g exactly, so dq = dk = 0, dv = sum over the
  group's heads of dY * sigmoid(G), dG = dY * V * sigmoid' (G);
* window >= S gives the global layer's gradients;
* a gate of +inf gives dG = 0 and the ungated layer's other gradients;
* rope_bwd is the transpose of the rotation (<R x, y> = <x, R^T y>);
* rms_norm_bwd matches finite differences of rms_norm on its own.
"""
import math

import numpy as np
import pytest

import oracle as orc


def _case(seed, B=1, S=7, Hq=4, Hkv=2, D=8, gated=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    g = rng.standard_normal((B, S, Hq, D)) if gated else None
    wq = 1.0 + 0.3 * rng.standard_normal(D)
    wk = 1.0 + 0.3 * rng.standard_normal(D)
    dy = rng.standard_normal((B, S, Hq, D))
    return q, k, v, g, wq, wk, dy


KW = dict(rope_dim=4, rope_theta=100.0, rms_eps=1e-3, pos_offset=5)


def _loss(q, k, v, g, wq, wk, dy, window, scale):
    y, _ = orc.attention_fwd(q, k, v, g, wq, wk, window=window, softmax_scale=scale, **KW)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("window,gated,scale", [(0, True, 0.0), (3, True, 0.0), (3, False, 0.7),
                                                (0, False, 0.0)])
def test_backward_matches_finite_differences(window, gated, scale):
    q, k, v, g, wq, wk, dy = _case(11 + window, gated=gated)
    grads = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=window, softmax_scale=scale, **KW)
    args = {"q": q, "k": k, "v": v, "gate": g, "wq": wq, "wk": wk}
    names = {"q": "dq", "k": "dk", "v": "dv", "gate": "dgate", "wq": "dq_norm_w", "wk": "dk_norm_w"}
    rng = np.random.default_rng(5)
    h = 1e-5
    for name, arr in args.items():
        if arr is None:
            assert grads[names[name]] is None
            continue
        flat = arr.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 40), replace=False)
        an = grads[names[name]].reshape(-1)
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp = _loss(q, k, v, g, wq, wk, dy, window, scale)
            flat[i] = old - h
            lm = _loss(q, k, v, g, wq, wk, dy, window, scale)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - an[i]) <= 1e-6 * max(1.0, abs(num)), (name, int(i), num, an[i])


def test_window_one_closed_form():
    q, k, v, g, wq, wk, dy = _case(3)
    r = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=1, **KW)
    assert np.max(np.abs(r["dq"])) < 1e-12 and np.max(np.abs(r["dk"])) < 1e-12
    assert np.max(np.abs(r["dq_norm_w"])) < 1e-12 and np.max(np.abs(r["dk_norm_w"])) < 1e-12
    sg = 1.0 / (1.0 + np.exp(-g))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    grp = Hq // Hkv
    vh = np.repeat(v, grp, axis=2)  # kv head of each query head
    dv = (dy * sg).reshape(B, S, Hkv, grp, D).sum(axis=3)
    np.testing.assert_allclose(r["dv"], dv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dgate"], dy * vh * sg * (1 - sg), rtol=1e-12, atol=1e-12)


def test_window_at_least_s_is_global():
    q, k, v, g, wq, wk, dy = _case(4)
    a = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=0, **KW)
    b = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=q.shape[1], **KW)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-13)


def test_gate_plus_inf_is_ungated():
    q, k, v, g, wq, wk, dy = _case(6)
    ginf = np.full_like(g, np.inf)
    a = orc.attention_bwd(q, k, v, ginf, wq, wk, dy, window=3, **KW)
    b = orc.attention_bwd(q, k, v, None, wq, wk, dy, window=3, **KW)
    assert np.all(a["dgate"] == 0.0)
    for key in ("dq", "dk", "dv", "dq_norm_w", "dk_norm_w"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-13)


def test_rope_bwd_is_the_transpose():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((9, 3, 16))
    y = rng.standard_normal((9, 3, 16))
    pos = np.arange(9) + 1000
    lhs = np.sum(orc.apply_partial_rope(x, pos, 10, 1e4) * y)
    rhs = np.sum(x * orc.rope_bwd(y, pos, 10, 1e4))
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_rms_norm_bwd_finite_differences():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 12))
    gam = 1.0 + 0.2 * rng.standard_normal(12)
    dxh = rng.standard_normal((5, 12))
    dx, dgam = orc.rms_norm_bwd(x, gam, 1e-2, dxh)
    h = 1e-6
    for i in range(5):
        for j in range(12):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            num = np.sum(dxh * (orc.rms_norm(xp, gam, 1e-2) - orc.rms_norm(xm, gam, 1e-2))) / (2 * h)
            assert abs(num - dx[i, j]) < 1e-7 * max(1.0, abs(num))
    for j in range(12):
        gp = gam.copy(); gp[j] += h
        gm = gam.copy(); gm[j] -= h
        num = np.sum(dxh * (orc.rms_norm(x, gp, 1e-2) - orc.rms_norm(x, gm, 1e-2))) / (2 * h)
        assert abs(num - dgam[j]) < 1e-7 * max(1.0, abs(num))


def test_backward_chunking_changes_nothing():
    q, k, v, g, wq, wk, dy = _case(10, S=23)
    a = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=5, chunk=1024, **KW)
    b = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=5, chunk=4, **KW)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [0, 5])
@pytest.mark.parametrize("gated", [True, False])
def test_backward_sampling_matches_full(window, gated):
    """rows / keys select entries of the full result: the same values (up to
    the order of the fp64 sums), and the row set grows to every row that sees
    a selected key (a key seen only by unselected rows is still right)."""
    q, k, v, g, wq, wk, dy = _case(11, B=2, S=29, gated=gated)
    full = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=window, chunk=6, **KW)
    rows = np.array([0, 3, 17, 28])
    keys = np.array([1, 2, 20, 27])
    for kw in (dict(rows=rows, keys=keys), dict(rows=rows), dict(keys=keys)):
        s = orc.attention_bwd(q, k, v, g, wq, wk, dy, window=window, chunk=3, **kw, **KW)
        r = kw.get("rows", np.arange(29))
        c = kw.get("keys", np.arange(29))
        np.testing.assert_allclose(s["dq"], full["dq"][:, r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s["dk"], full["dk"][:, c], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s["dv"], full["dv"][:, c], rtol=1e-12, atol=1e-12)
        if gated:
            np.testing.assert_allclose(s["dgate"], full["dgate"][:, r], rtol=1e-12, atol=1e-12)
        assert s["dq_norm_w"] is None and s["dk_norm_w"] is None
