"""Pins of the oracle's readout backward (FreeSolo Sec. 3.3 "Training": gradients
flow through the selected tokens only, none through the indices; App. D.4).

The backward is pinned to things other than itself:
  * central finite differences of the oracle's FORWARD readout (a separate C
    function, oracle_readout) with the selection held fixed;
  * invariants that hold for any input: the softmax gradient sums to zero over
    the selected tokens (so the key gradients do); at eps = 0 the RMSNorm output
    does not change when u is scaled (so sum_j dv_j . v_j = 0); the output is
    linear in the gain (so dg . g = dout . o); the whole backward is linear in dout;
  * special cases: one selected token gives no query or key gradient and
    dv = the RMSNorm backward of dout; an empty selection gives no gradient at all;
  * tokens outside the selection receive nothing.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng


def _head(N=256, d=16, seed=0, scale=1.0):
    r = RNG(seed)
    q = r.standard_normal((N, d)) * scale
    k = r.standard_normal((N, d)) * scale
    v = r.standard_normal((N, d))
    return q, k, v


def _loss(q, k, v, g, sel, dout, prm, i_lo):
    """sum_i dout_i . o_i with the forward readout."""
    tot = 0.0
    for r, cells in enumerate(sel):
        tot += float(dout[r] @ oracle.readout(q[i_lo + r], k, v, list(cells), g, prm))
    return tot


def _fd(f, x, idx, h=1e-6):
    x0 = x[idx]
    x[idx] = x0 + h
    fp = f()
    x[idx] = x0 - h
    fm = f()
    x[idx] = x0
    return (fp - fm) / (2 * h)


@pytest.mark.parametrize("s,K,d,gain", [(4, 3, 8, False), (8, 4, 16, True), (1, 5, 6, True)])
def test_backward_matches_finite_differences(s, K, d, gain):
    """Every gradient entry against a central difference of the forward readout."""
    N = 64
    prm = oracle.Params(s=s, B=16, K=K, eps=1e-6)
    q, k, v = _head(N, d, seed=s * 10 + K)
    r = RNG(7 + d)
    g = r.uniform(0.5, 1.5, d) if gain else None
    M = N // s
    i_lo, n = 40, 3
    sel = np.full((n, K), -1, np.int32)
    for row in range(n):
        cells = r.choice(M, size=K - (row % 2), replace=False)  # one row with a -1 pad
        sel[row, :len(cells)] = cells
    dout = r.standard_normal((n, d))
    res = oracle.backward(q, k, v, sel, dout, g, prm, i_lo, i_lo + n)
    f = lambda: _loss(q, k, v, g, sel, dout, prm, i_lo)
    tol = dict(rtol=2e-6, atol=2e-7)
    for row in range(n):
        for c in range(d):
            np.testing.assert_allclose(res["dq"][row, c], _fd(f, q, (i_lo + row, c)), **tol)
    toks = sorted({j for row in sel for c in row if c >= 0 for j in range(c * s, (c + 1) * s)})
    for j in toks[:: max(1, len(toks) // 12)]:
        for c in range(0, d, 3):
            np.testing.assert_allclose(res["dk"][j, c], _fd(f, k, (j, c)), **tol)
            np.testing.assert_allclose(res["dv"][j, c], _fd(f, v, (j, c)), **tol)
    if gain:
        for c in range(d):
            np.testing.assert_allclose(res["dg"][c], _fd(f, g, c), **tol)


def test_unselected_tokens_receive_nothing():
    """No gradient reaches a token outside the selection (and none flows through the
    indices: the selection is an input)."""
    prm = oracle.Params(s=4, B=16, K=2)
    q, k, v = _head(64, 8, seed=3)
    sel = np.array([[2, 9], [9, -1]], np.int32)
    dout = RNG(1).standard_normal((2, 8))
    res = oracle.backward(q, k, v, sel, dout, None, prm, 50, 52)
    hit = np.zeros(64, bool)
    for c in (2, 9):
        hit[c * 4:(c + 1) * 4] = True
    assert np.all(res["dk"][~hit] == 0) and np.all(res["dv"][~hit] == 0)
    assert np.all(np.abs(res["dv"][hit]).sum(axis=1) > 0)


def test_key_gradients_sum_to_zero():
    """The softmax gradient sums to zero over the selected tokens, so for one query the
    key gradients over its tokens sum to zero."""
    prm = oracle.Params(s=8, B=32, K=4)
    q, k, v = _head(256, 16, seed=5, scale=0.7)
    sel = np.array([[1, 5, 11, 20]], np.int32)
    res = oracle.backward(q, k, v, sel, RNG(2).standard_normal((1, 16)), None, prm, 200, 201)
    assert np.abs(res["dk"].sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(res["dk"]).max())
    assert np.abs(res["dk"]).max() > 1e-3


def test_rmsnorm_scale_invariance():
    """At eps = 0 the output does not change when u is scaled, so du . u = 0, that is
    sum_j dv_j . v_j = 0; with eps > 0 it is not zero."""
    q, k, v = _head(128, 12, seed=9)
    sel = np.array([[0, 3, 7]], np.int32)
    dout = RNG(4).standard_normal((1, 12))
    res = oracle.backward(q, k, v, sel, dout, RNG(5).uniform(0.5, 2, 12), oracle.Params(s=4, B=16, K=3, eps=0.0),
                          100, 101)
    assert abs(np.sum(res["dv"] * v)) < 1e-12 * np.abs(res["dv"]).sum() * np.abs(v).max()
    res = oracle.backward(q, k, v, sel, dout, None, oracle.Params(s=4, B=16, K=3, eps=0.5), 100, 101)
    assert abs(np.sum(res["dv"] * v)) > 1e-3


def test_gain_gradient_closed_form():
    """o is linear in g, so dg . g = dout . o (summed over the queries)."""
    prm = oracle.Params(s=4, B=16, K=3)
    q, k, v = _head(128, 10, seed=11)
    g = RNG(6).uniform(0.2, 3.0, 10)
    sel = np.array([[0, 4, 9], [2, -1, -1], [5, 6, 7]], np.int32)
    dout = RNG(8).standard_normal((3, 10))
    res = oracle.backward(q, k, v, sel, dout, g, prm, 90, 93)
    want = sum(float(dout[r] @ oracle.readout(q[90 + r], k, v, list(sel[r]), g, prm)) for r in range(3))
    np.testing.assert_allclose(res["dg"] @ g, want, rtol=1e-12)


def test_single_token_closed_form():
    """s = 1, K = 1: p = 1, u = v_j, so no query or key gradient, and dv_j is the RMSNorm
    backward r g dout - (r^3/d)(sum g dout v_j) v_j written out here."""
    d = 9
    prm = oracle.Params(s=1, B=8, K=1, eps=1e-3)
    q, k, v = _head(32, d, seed=13)
    g = RNG(9).uniform(0.5, 1.5, d)
    dout = RNG(10).standard_normal((1, d))
    res = oracle.backward(q, k, v, np.array([[6]], np.int32), dout, g, prm, 20, 21)
    u = v[6]
    r = 1.0 / np.sqrt(np.mean(u * u) + 1e-3)
    want = r * g * dout[0] - r ** 3 / d * np.sum(g * dout[0] * u) * u
    assert np.all(res["dq"] == 0) and np.all(res["dk"] == 0)
    np.testing.assert_allclose(res["dv"][6], want, rtol=1e-13)
    np.testing.assert_allclose(res["dg"], r * dout[0] * u, rtol=1e-13)


def test_empty_selection_gives_no_gradient():
    prm = oracle.Params(s=4, B=16, K=3)
    q, k, v = _head(64, 8, seed=15)
    res = oracle.backward(q, k, v, np.full((2, 3), -1, np.int32), np.ones((2, 8)), np.ones(8), prm, 10, 12)
    for x in ("dq", "dk", "dv", "dg"):
        assert np.all(res[x] == 0)


def test_backward_linear_in_dout():
    prm = oracle.Params(s=4, B=16, K=3)
    q, k, v = _head(128, 8, seed=17)
    sel = np.array([[1, 8, 20], [3, 4, -1]], np.int32)
    a, b = RNG(11).standard_normal((2, 8)), RNG(12).standard_normal((2, 8))
    ra = oracle.backward(q, k, v, sel, a, None, prm, 100, 102)
    rb = oracle.backward(q, k, v, sel, b, None, prm, 100, 102)
    rab = oracle.backward(q, k, v, sel, 2 * a - 3 * b, None, prm, 100, 102)
    for x in ("dq", "dk", "dv", "dg"):
        np.testing.assert_allclose(rab[x], 2 * ra[x] - 3 * rb[x], atol=1e-12)


def test_abs_sizes_bound_the_gradients():
    """The term sizes bound the gradients entry by entry (|sum| <= sum of |terms|)."""
    prm = oracle.Params(s=4, B=16, K=4)
    q, k, v = _head(128, 8, seed=19)
    sel = np.array([[0, 5, 9, 13], [2, 3, 4, 30]], np.int32)
    res = oracle.backward(q, k, v, sel, RNG(13).standard_normal((2, 8)), RNG(14).uniform(0.5, 2, 8), prm, 124, 126,
                          want_abs=True)
    for x in ("dq", "dk", "dv", "dg"):
        assert np.all(np.abs(res[x]) <= res[x + "_abs"] * (1 + 1e-12) + 1e-300)
    assert np.all(res["dq_abs"] > 0)


def test_backward_rejects_a_cell_past_the_end():
    prm = oracle.Params(s=4, B=16, K=2)
    q, k, v = _head(64, 8, seed=21)
    with pytest.raises(ValueError):
        oracle.backward(q, k, v, np.array([[16, -1]], np.int32), np.ones((1, 8)), None, prm, 60, 61)


def test_sizes_widen_where_u_cancels():
    """With q = 0 the softmax is uniform (p = 1/4 over a 4-token cell); values v, -v, w,
    -w + c give u = c / 4, far smaller than its terms.  Rounding p_j v_j and their sum
    leaves u off by about e sum_j p_j |v_j| rather than e |u|, so dg = r dout u is off by
    about e r |dout| sum_j p_j |v_j|: the error scale of dg must be at least that (here
    ~1000 |dg|).  Without cancellation it stays comparable to |dg|."""
    d, s = 4, 4
    prm = oracle.Params(s=s, B=8, K=1, eps=1.0)
    q = np.zeros((16, d))
    k = RNG(20).standard_normal((16, d))
    a = np.array([1.0, -2.0, 0.5, 3.0]) * 100.0
    b = np.array([-1.5, 1.0, 2.0, -0.5]) * 100.0
    c = np.array([0.3, 0.2, -0.1, 0.4])
    v = np.zeros((16, d))
    v[8:12] = [a, -a, b, -b + c]
    dout = np.array([[1.0, -2.0, 0.5, 1.5]])
    res = oracle.backward(q, k, v, np.array([[2]], np.int32), dout, None, prm, 12, 13, want_abs=True)
    u = c / 4
    r = 1.0 / np.sqrt(np.mean(u * u) + 1.0)
    spread = np.abs(v[8:12]).sum(axis=0) / 4
    assert np.all(res["dg_abs"] >= r * np.abs(dout[0]) * spread * (1 - 1e-12))
    assert np.all(res["dg_abs"] > 100.0 * np.abs(res["dg"]))
    v[8:12] = [a, a, b, b]  # no cancellation
    res = oracle.backward(q, k, v, np.array([[2]], np.int32), dout, None, prm, 12, 13, want_abs=True)
    assert np.all(res["dg_abs"] < 10.0 * np.abs(res["dg"]))
