"""The comparison rules of the GPU parity tests, exercised on the CPU.

A near-tie makes several selections correct; the parity helpers must accept
every correct one (and read it out with the oracle) and still reject a wrong
one.  The cases plant exact ties with the oracle's own inputs: two cells with
identical keys far behind the query score identically in Eq. 7 (the prior has
saturated to exactly 1 in fp64), and two cells with identical key norms tie in
the TopP order of Eq. 8.
"""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import oracle
from tests import parity_utils as pu


def _tied_scores(K=1):
    g = np.random.default_rng(5)
    N, d = 1024, 8
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    k[2 * 32:3 * 32] = 6.0 * g.normal(size=(32, d))   # cell 2: by far the largest norms
    k[5 * 32:6 * 32] = k[2 * 32:3 * 32]               # cell 5: the same keys
    p = fsl.Params(P=64, W=8, K=K)
    op = pu.oracle_params(p)
    ref = pu.attach(oracle.head(q, k, v, None, op), (q, k, v, None), op)
    return p, ref


def test_exact_tie_other_choice_accepted():
    p, ref = _tied_scores()
    rows = np.nonzero(ref["gap_k"] == 0.0)[0]
    assert len(rows) > 100 and np.all(ref["sel"][rows, 0] == 2)  # the smaller id wins the tie
    sel = ref["sel"].copy()
    out = ref["out"].copy()
    for r in rows:  # a GPU that broke the tie the other way
        sel[r, 0] = 5
        out[r] = oracle.readout(ref["inputs"][0][r], ref["inputs"][1], ref["inputs"][2], [5], None, ref["prm"])
    exact, ties = pu.compare_head(sel, out.astype(np.float32), ref, p, "f32", what="tie")
    assert ties >= len(rows) and exact + ties == len(sel)


def test_exact_tie_wrong_output_rejected():
    p, ref = _tied_scores()
    r = int(np.nonzero(ref["gap_k"] == 0.0)[0][0])
    sel = ref["sel"].copy()
    sel[r, 0] = 5
    with pytest.raises(AssertionError, match="fp32 output error"):  # output of cell 2 kept with cell 5 chosen
        pu.compare_head(sel, ref["out"].astype(np.float32), ref, p, "f32", what="tie")


def test_near_tie_wrong_cell_rejected():
    p, ref = _tied_scores()
    r = int(np.nonzero(ref["gap_k"] == 0.0)[0][0])
    A = ref["retained"][r // 128][: ref["n_ret"][r // 128]]
    low = int([c for c in A if c not in (2, 5)][0])  # a cell far below the tied pair
    sel = ref["sel"].copy()
    sel[r, 0] = low
    out = ref["out"].copy()
    out[r] = oracle.readout(ref["inputs"][0][r], ref["inputs"][1], ref["inputs"][2], [low], None, ref["prm"])
    with pytest.raises(AssertionError, match="outranks"):
        pu.compare_head(sel, out.astype(np.float32), ref, p, "f32", what="tie")


def test_exact_selection_mismatch_rejected():
    p, ref = _tied_scores(K=2)
    r = int(np.nonzero(ref["gap_k"] > 1e-3)[0][-1])
    sel = ref["sel"].copy()
    sel[r] = sel[r][::-1]
    with pytest.raises(AssertionError, match="selection differs"):
        pu.compare_head(sel, ref["out"].astype(np.float32), ref, p, "f32", what="exact")


def test_topp_boundary_tie_validated():
    """Equal norms at the P-th place: either cell may be retained, never a lower one."""
    a = np.array([5.0, 9.0, 4.0, 7.0, 7.0, 1.0, 3.0, 2.0])  # P = 2: 9, then 7 (cell 3) tied with 7 (cell 4)
    P, W, n = 2, 2, 8
    assert pu.boundary_pool(a, n, P) == {3, 4}
    pu.check_retained_valid([1, 3, 6, 7], a, n, P, W)  # the oracle's choice
    pu.check_retained_valid([1, 4, 6, 7], a, n, P, W)  # the other correct one
    with pytest.raises(AssertionError):
        pu.check_retained_valid([1, 0, 6, 7], a, n, P, W)  # cell 0 (norm 5) is below the boundary
    with pytest.raises(AssertionError):
        pu.check_retained_valid([1, 3, 6], a, n, P, W)     # Recent_W incomplete


# ---- the readout backward's bar (tests/test_gpu_backward.py) ---------------------------

def _bf16(x):
    """Round fp32 values to bf16 (nearest even), returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _split(x, with_lo):
    hi = _bf16(x)
    return (hi, _bf16(x - hi)) if with_lo else (hi, np.zeros_like(hi))


def _emulated_backward(q, k, v, sel, dout, s, with_lo):
    """fp32 emulation of one head's readout backward with the matrix-product operands
    that are not exact bf16 values (p, du, dS) split into bf16 hi + lo parts (or, with
    with_lo False, rounded to bf16 alone); q, k, v, dout are exact bf16 values."""
    f32 = np.float32
    N, d = k.shape
    dq = np.zeros((len(sel), d), f32)
    dk = np.zeros((N, d), f32)
    dv = np.zeros((N, d), f32)
    sd = f32(np.sqrt(d))
    for r, cells in enumerate(sel):
        toks = np.array([c * s + x for c in cells if c >= 0 for x in range(s)], np.int64)
        if len(toks) == 0:
            continue
        qi = q[r].astype(f32)
        K, V = k[toks].astype(f32), v[toks].astype(f32)
        lg = (K @ qi) / sd
        p = np.exp(lg - lg.max()).astype(f32)
        p = (p / p.sum()).astype(f32)
        ph, pl = _split(p, with_lo)
        u = (ph @ V + pl @ V).astype(f32)
        rn = f32(1.0) / np.sqrt(f32(np.mean(u * u)) + f32(1e-8))
        du = (rn * dout[r] - rn ** 3 / d * f32(np.sum(dout[r] * u)) * u).astype(f32)
        uh, ul = _split(du, with_lo)
        dp = (V @ uh + V @ ul).astype(f32)
        ds = (p * (dp - f32(du @ u))).astype(f32)
        sh, sl = _split(ds, with_lo)
        dq[r] = (sh @ K + sl @ K) / sd
        dk[toks] += (np.outer(sh, qi) + np.outer(sl, qi)) / sd
        dv[toks] += np.outer(ph, uh) + np.outer(ph, ul) + np.outer(pl, uh)
    return dq, dk, dv


def _beyond_bar(got, ref, scale):
    return int(pu.bwd_beyond_bar(got, ref, scale, "bf16").sum())


def test_backward_bar_admits_split_products_and_rejects_bf16_only():
    """The bf16 bar of the readout backward (2^-16 of the oracle's error scale) is met by
    fp32 arithmetic whose non-bf16 product operands keep a lo part, and is missed when
    the lo parts are dropped (operands rounded to bf16 alone, ~2^-9 of their size)."""
    import synth
    w = synth.Workload(batch=1, H=1, N=768, d=64, dtype="bf16", seed=77, needle_frac=0.01)
    f64 = {x: synth.to_f64(synth.tensor(w, x)[0, 0], "bf16") for x in ("q", "k", "v", "dout")}
    rng = np.random.default_rng(5)
    i_lo = 384
    sel = np.full((w.N - i_lo, 4), -1, np.int32)
    for r in range(len(sel)):
        n = ((i_lo + r) // 128) * 4
        sel[r] = rng.choice(n, size=4, replace=False)
    ref = oracle.backward(f64["q"], f64["k"], f64["v"], sel, f64["dout"][i_lo:], None, oracle.Params(), i_lo, w.N,
                          want_abs=True)
    args = (f64["q"][i_lo:].astype(np.float32), f64["k"].astype(np.float32), f64["v"].astype(np.float32), sel,
            f64["dout"][i_lo:].astype(np.float32), 32)
    good = _emulated_backward(*args, with_lo=True)
    bad = _emulated_backward(*args, with_lo=False)
    for name, g, b_ in zip(("dq", "dk", "dv"), good, bad):
        assert _beyond_bar(g, ref[name], ref[name + "_abs"]) == 0, name
        assert _beyond_bar(b_, ref[name], ref[name + "_abs"]) > 0, name
