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
