"""Pins of the oracle's projections (linear, qkvg_proj).

The projection is a plain definition (y = x W^T), so its pins are a worked
example by hand, identity and permutation weights, linearity, and the
head layout of the fused projection's four parts."""

import numpy as np

import oracle as orc


def test_hand_worked_example():
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])
    # rows of y: (x.w_0, x.w_1, x.w_2, x.w_3)
    want = np.array([[1.0, 2.0, 3.0, 0.0], [3.0, 4.0, 7.0, 2.0]])
    assert np.array_equal(orc.linear(x, w), want)


def test_identity_and_permutation_weights():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7))
    assert np.array_equal(orc.linear(x, np.eye(7)), x)
    perm = rng.permutation(7)
    # row j of the weight picks input feature perm[j]
    assert np.array_equal(orc.linear(x, np.eye(7)[perm]), x[:, perm])


def test_linearity():
    rng = np.random.default_rng(2)
    x1, x2 = rng.standard_normal((2, 6, 9))
    w = rng.standard_normal((4, 9))
    lhs = orc.linear(2.5 * x1 - 0.5 * x2, w)
    rhs = 2.5 * orc.linear(x1, w) - 0.5 * orc.linear(x2, w)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_qkvg_layout_and_split():
    """With a weight whose row r is the one-hot e_(r mod in), the output
    column of head h, dim d of each part is input feature (row index) mod in,
    so the split and the head reshape can be checked entry by entry."""
    Hq, Hkv, D, T = 4, 2, 3, 2
    nq, nk = Hq * D, Hkv * D
    n_in = 5
    for gated in (True, False):
        n_out = 2 * nq + 2 * nk if gated else nq + 2 * nk
        w = np.zeros((n_out, n_in))
        w[np.arange(n_out), np.arange(n_out) % n_in] = 1.0
        x = np.arange(T * n_in, dtype=np.float64).reshape(T, n_in) + 1.0
        q, k, v, g = orc.qkvg_proj(x, w, Hq, Hkv, D, gated)
        assert q.shape == (T, Hq, D) and k.shape == (T, Hkv, D) and v.shape == (T, Hkv, D)
        for t in range(T):
            for h in range(Hq):
                for d in range(D):
                    assert q[t, h, d] == x[t, (h * D + d) % n_in]
                    if gated:
                        assert g[t, h, d] == x[t, (nq + 2 * nk + h * D + d) % n_in]
            for h in range(Hkv):
                for d in range(D):
                    assert k[t, h, d] == x[t, (nq + h * D + d) % n_in]
                    assert v[t, h, d] == x[t, (nq + nk + h * D + d) % n_in]
        assert (g is None) == (not gated)
