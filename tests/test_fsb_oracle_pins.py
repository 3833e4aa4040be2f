"""Pins of the FS-B oracle (FreeSolo, Sec. 3.4 "Balanced tree search (FS-B)";
App. E.1 "Streaming forests") against what the page and mathematics fix.

None of these re-types the oracle's formulas: each checks a value the page prints
(the 13 = 8 + 4 + 1 forest of Figure 9), a property it states (balanced chunk
trees, height ceil(log2 M), fewer than 2M nodes, enclosing balls at join nodes,
U_v bounding Eq. 7 below v for c >= 1, the second forest's admission by a_c >=
tau), a closed form (collinear mean keys split at their median; Eq. 12 equals
Eq. 7 on one-token cells), or an invariant (exhaustive search when the beam
holds every cell; causality).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import FsbParams, Params


def rng(seed):
    return np.random.default_rng(seed)


def data(seed, N, d, scale=1.0):
    g = rng(seed)
    q = g.normal(size=(N, d))
    k = g.normal(size=(N, d)) * g.lognormal(sigma=0.5, size=(N, 1)) * scale
    v = g.normal(size=(N, d))
    return q, k, v


def depths(F):
    dep = {F["root"]: 0}
    stack = [F["root"]]
    while stack:
        x = stack.pop()
        for ch in (F["left"][x], F["right"][x]):
            if ch >= 0:
                dep[ch] = dep[x] + 1
                stack.append(ch)
    return dep


def leaves_below(F, x):
    if F["cell"][x] >= 0:
        return [int(F["cell"][x])]
    return leaves_below(F, F["left"][x]) + leaves_below(F, F["right"][x])


# ---------------------------------------------------------- App. E.1 "Chunks" ----

def test_chunk_decomposition_figure9():
    """Eq. 18 and Figure 9: 13 = 8 + 4 + 1, older cells in larger chunks; the 13-cell
    forest has height ceil(log2 13) = 4."""
    assert oracle.fsb_chunks(13) == [8, 4, 1]
    assert oracle.fsb_chunks(512) == [512]
    assert oracle.fsb_chunks(0) == []
    assert oracle.fsb_chunks(127) == [64, 32, 16, 8, 4, 2, 1]
    _, k, _ = data(1, 13 * 32, 8)
    kbar, a = oracle.cell_summaries(k)
    F = oracle.fsb_forest(kbar, a, np.arange(13))
    dep = depths(F)
    assert max(dep[x] for x in dep if F["cell"][x] >= 0) == 4
    # the chunks' cells: {c1..c8}, {c9..c12}, {c13} are the root's subtrees along the join chain
    root = F["root"]
    assert sorted(leaves_below(F, F["left"][root])) == list(range(8))
    J2 = F["right"][root]
    assert sorted(leaves_below(F, F["left"][J2])) == list(range(8, 12))
    assert leaves_below(F, F["right"][J2]) == [12]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 13, 16, 33, 100, 127, 128])
def test_forest_shape(M):
    """Every chunk of 2^k cells is a perfect binary tree of height k (median splits of the
    content order); the forest has height ceil(log2 M), fewer than 2M nodes, and its leaves
    are the admitted cells, each once."""
    _, k, _ = data(2 + M, M * 32, 8)
    kbar, a = oracle.cell_summaries(k)
    cells = np.arange(M)
    F = oracle.fsb_forest(kbar, a, cells)
    assert len(F["count"]) == 2 * M - 1 < 2 * M
    dep = depths(F)
    leaf_depth = [dep[x] for x in dep if F["cell"][x] >= 0]
    assert max(leaf_depth) == math.ceil(math.log2(M)) if M > 1 else max(leaf_depth) == 0
    assert sorted(leaves_below(F, F["root"])) == list(cells)
    for x in range(len(F["count"])):
        if F["cell"][x] < 0:
            l, r = F["left"][x], F["right"][x]
            assert F["count"][x] == F["count"][l] + F["count"][r]
    # chunk roots: the root's left subtrees along the join chain, sizes as Eq. 18
    node, sizes = F["root"], []
    for size in oracle.fsb_chunks(M)[:-1]:
        sizes.append(F["count"][F["left"][node]])
        sub = F["left"][node]
        sd = {x: dep[x] - dep[sub] for x in dep}
        below = leaves_below(F, sub)
        assert all(sd[x] == int(math.log2(size)) for x in range(len(F["count"])) if F["cell"][x] in below)
        node = F["right"][node]
    sizes.append(F["count"][node])
    assert sizes == oracle.fsb_chunks(M)


# -------------------------------------------------- App. E.1 "Node summaries" ----

def test_node_summaries_and_enclosing_balls():
    """Eq. 20: mu_v is the mean of the cell means below v, A_v their largest norm, p_v^min
    the earliest centre; rho_v is their largest distance from mu_v in a chunk tree, and at a
    join node (Eq. 21) a radius whose ball still encloses every cell mean below (the
    triangle inequality), which is what keeps Eq. 11 an upper bound there."""
    _, k, _ = data(3, 45 * 32, 12)
    kbar, a = oracle.cell_summaries(k)
    cells = np.arange(45)  # 45 = 32 + 8 + 4 + 1: three join nodes
    F = oracle.fsb_forest(kbar, a, cells)
    joins = 0
    for x in range(len(F["count"])):
        below = leaves_below(F, x)
        np.testing.assert_allclose(F["mu"][x], kbar[below].mean(0), rtol=1e-12, atol=1e-14)
        assert F["A"][x] == a[below].max()
        assert F["pmin"][x] == (min(below) + 0.5) * 32
        far = max(np.linalg.norm(kbar[c] - F["mu"][x]) for c in below)
        assert F["rho"][x] >= far - 1e-12
        # chunk-tree nodes carry the exact radius; join nodes the looser Eq. 21 bound
        is_join = F["cell"][x] < 0 and F["count"][F["left"][x]] != F["count"][F["right"][x]]
        joins += is_join
        if not is_join:
            assert F["rho"][x] == pytest.approx(far, rel=1e-12, abs=1e-14)
    assert joins == 3


def test_collinear_split_closed_form():
    """Mean keys on one line, kbar_c = m + t_c e: the centred means are all parallel to e, so
    the power iteration returns +-e (the sign of the farthest cell's offset) and the split is
    at the median of t: the first half of the chunk (by projection, ascending) goes left."""
    d, n = 6, 16
    g = rng(4)
    e = g.normal(size=d); e /= np.linalg.norm(e)
    m = g.normal(size=d)
    t = g.permutation(np.linspace(-3.0, 5.0, n))  # distinct; the farthest from their mean (1.0) is t = 5
    kbar = m[None, :] + t[:, None] * e[None, :]
    a = np.ones(n)
    F = oracle.fsb_forest(kbar, a, np.arange(n))
    left = sorted(leaves_below(F, F["left"][F["root"]]))
    assert left == sorted(np.argsort(t)[: n // 2].tolist())  # u = +e: the smaller t go left
    # the farthest cell on the negative side flips u, and with it the halves
    t2 = -t
    kbar2 = m[None, :] + t2[:, None] * e[None, :]
    F2 = oracle.fsb_forest(kbar2, a, np.arange(n))
    assert sorted(leaves_below(F2, F2["left"][F2["root"]])) == sorted(np.argsort(-t2)[: n // 2].tolist())


# ---------------------------------------------------------------- Eq. 11 ----

@pytest.mark.parametrize("c,lam", [(1.0, 1.0), (8.0, 1.0), (1.0, 0.0), (3.0, 0.25)])
def test_priority_bounds_cell_scores(c, lam):
    """Sec. 3.4: for c >= 1, U_v bounds the Eq. 7 score of every cell below v (the radius
    bounds the content term; A_v and p_v^min bound the nonnegative, monotone prior).  Checked
    for every node of a 70-cell forest and queries of the first block that has all 70 cells
    available (positions 2304 .. 2431, so every prior offset i - p_c is positive)."""
    N, d = 19 * 128, 16
    q, k, _ = data(5, N, d)
    kbar, a = oracle.cell_summaries(k)
    prm, fb = Params(lam=lam), FsbParams(c=c)
    F = oracle.fsb_forest(kbar, a, np.arange(70))
    for i in range(18 * 128, N, 17):
        for x in range(len(F["count"])):
            U = oracle.fsb_node_priority(q[i], i, F["mu"][x], F["rho"][x], F["A"][x], F["pmin"][x], prm, fb)
            for cell in leaves_below(F, x):
                assert U >= oracle.cell_score(q[i], kbar[cell], a[cell], i, cell, prm) - 1e-10


def test_leaf_priority_is_the_cell_score():
    """A leaf holds one cell: mu = kbar_c, rho = 0, A = a_c, p^min = p_c, so Eq. 11 is Eq. 7."""
    N, d = 20 * 32, 8
    q, k, _ = data(6, N, d)
    kbar, a = oracle.cell_summaries(k)
    for c in (0, 7, 19):
        for i in (20 * 32 - 1, 600):
            U = oracle.fsb_node_priority(q[i], i, kbar[c], 0.0, a[c], (c + 0.5) * 32, Params(), FsbParams())
            assert U == pytest.approx(oracle.cell_score(q[i], kbar[c], a[c], i, c, Params()), rel=1e-13)


# ------------------------------------------------------------ beam search ----

def test_beam_holding_every_cell_is_exhaustive():
    """With W^b at least the number of cells, no node is ever dropped: both candidate sets
    are the whole admitted prefix, so B_i = C_i (the union of the two forests' leaves)."""
    N, d = 1024, 8
    q, k, v = data(7, N, d)
    res = oracle.fsb_head(q, k, v, prm=Params(), fb=FsbParams(tau=1e300, Wb=64))
    for i in range(128, N, 41):
        n_avail = (i // 128) * 4
        assert res["n_cand"][i] == n_avail
        assert list(res["cand"][i][:n_avail]) == list(range(n_avail))
    assert np.all(res["gap_beam"][128:] == np.inf)


def test_leaf_keeps_its_slot():
    """App. E.1: a leaf reached early on a short branch keeps its slot.  17 = 16 + 1 cells:
    the 17th cell is a leaf right under the root.  With W^b = 2 and that cell made the
    least attractive of all, it is still among the candidates, next to one leaf of the
    16-cell chunk.  (B = s = 32 here, so that a block sees exactly 17 cells.)"""
    N, d = 18 * 32, 8
    q, k, v = data(8, N, d)
    k[16 * 32:17 * 32] = 1e-3 * np.abs(k[16 * 32:17 * 32]) * -np.sign(q[N - 1])  # tiny norm, against the query
    prm = Params(B=32)
    res = oracle.fsb_head(q, k, v, prm=prm, fb=FsbParams(tau=1e300, Wb=2), i_lo=N - 1, i_hi=N)
    cand = [c for c in res["cand"][0] if c >= 0]
    assert 16 in cand and len(cand) == 2
    # the cell is the least attractive: with a beam that holds everything it comes last
    full = oracle.fsb_head(q, k, v, prm=prm, fb=FsbParams(tau=1e300, Wb=32), i_lo=N - 1, i_hi=N)
    kbar, a = full["kbar"], full["a"]
    r = [oracle.cell_score(q[N - 1], kbar[c], a[c], N - 1, c, prm) for c in range(17)]
    assert int(np.argmin(r)) == 16


def test_second_forest_admits_at_threshold():
    """Eq. 10: the second forest admits c with a_c >= tau.  With tau equal to the largest
    cell norm only that cell is admitted; with a beam of one, the candidates are forest 0's
    leaf plus that cell.  (Content-only routing, lambda = 0, so that forest 0's single slot
    does not go to the largest-norm cell anyway.)"""
    N, d = 1024, 8
    q, k, v = data(9, N, d)
    kbar, a = oracle.cell_summaries(k)
    i = N - 1
    n_avail = (i // 128) * 4
    top = int(np.argmax(a[:n_avail]))
    prm = Params(lam=0.0)
    lo = i - 127  # the last block's queries
    res = oracle.fsb_head(q, k, v, prm=prm, fb=FsbParams(tau=float(a[top]), Wb=1), i_lo=lo, i_hi=i + 1)
    res0 = oracle.fsb_head(q, k, v, prm=prm, fb=FsbParams(tau=1e300, Wb=1), i_lo=lo, i_hi=i + 1)
    resz = oracle.fsb_head(q, k, v, prm=prm, fb=FsbParams(tau=0.0, Wb=1), i_lo=lo, i_hi=i + 1)
    other = 0
    for r in range(128):
        cand = [c for c in res["cand"][r] if c >= 0]
        only0 = [c for c in res0["cand"][r] if c >= 0]
        assert len(only0) == 1
        assert top in cand and set(cand) == set(only0) | {top}
        other += top not in only0
        # tau = 0 admits everything: both forests are the same, the union adds nothing
        assert [c for c in resz["cand"][r] if c >= 0] == only0
    assert other > 10  # queries whose forest-0 leaf is another cell


# ---------------------------------------------------------------- Eq. 12 ----

def test_rerank_one_token_cells_is_eq7():
    """With one token per cell (s = 1) the log-sum-exp of Eq. 12 is that token's logit, the
    cell mean is the key and a_c its norm: the reranked score is exactly Eq. 7's."""
    N, d = 64, 8
    q, k, _ = data(10, N, d)
    prm = Params(s=1, B=4)
    kbar, a = oracle.cell_summaries(k, prm)
    for i, c in [(40, 3), (63, 50), (12, 11)]:
        r, _ = oracle.fsb_rerank_score(q[i], k, a[c], i, c, prm)
        assert r == pytest.approx(oracle.cell_score(q[i], kbar[c], a[c], i, c, prm), rel=1e-13, abs=1e-13)


def test_rerank_gap_closed_form():
    """The near-tie gap of the rerank: the smallest gap of adjacent scores among the K + 1
    best, each against the larger of the two scores' term sizes.  One-token cells (s = 1),
    content-only scores of cells (3, -2), (0.5, 0.4), (-1, -1), (0.1, 0) for q = (1, 1):
    1, 0.9, -2, 0.1 (times 1/sqrt 2) with sizes 5, 0.9, 2, 0.1.  K = 2: the pairs (1, 0.9)
    and (0.9, 0.1) give min(0.1 / 5, 0.8 / 0.9) = 0.02; K = 3 adds (0.1, -2): 2.1 / 2."""
    d = 2
    k = np.array([[3.0, -2.0], [0.5, 0.4], [-1.0, -1.0], [0.1, 0.0], [0.0, 0.0], [0.0, 0.0], [0.0, 0.0],
                  [0.0, 0.0]])
    q = np.tile([1.0, 1.0], (len(k), 1))
    for K, expect in ((2, 0.1 / 5.0), (1, 0.1 / 5.0), (3, 0.1 / 5.0)):
        res = oracle.fsb_head(q, k, np.zeros_like(k), prm=Params(s=1, B=4, K=K, lam=0.0),
                              fb=FsbParams(tau=1e300, Wb=8), i_lo=4, i_hi=5, want_out=False)
        assert list(res["sel"][0][:K]) == [0, 1, 3][:K]
        assert res["gap_rerank"][0] == pytest.approx(expect, rel=1e-13)
    # a second query with the order decided by the lower pair only: cells 1 and 3 selected
    # (K = 2 from the candidates {1, 2, 3} of a forest without cell 0): pairs (0.9, 0.1) and
    # (0.1, -2) -> min(0.8 / 0.9, 2.1 / 2)
    k2 = k.copy()
    k2[0] = [-30.0, -30.0]
    res = oracle.fsb_head(q, k2, np.zeros_like(k2), prm=Params(s=1, B=4, K=2, lam=0.0),
                          fb=FsbParams(tau=1e300, Wb=8), i_lo=4, i_hi=5, want_out=False)
    assert list(res["sel"][0]) == [1, 3]
    assert res["gap_rerank"][0] == pytest.approx(0.8 / 0.9, rel=1e-13)


def test_rerank_log_sum_exp_closed_forms():
    """Identical tokens in a cell: LSE = l + log(s).  Two distinct logits: log(e^x + e^y) in
    closed form, finite even for logits near 1000 (a stable log-sum-exp)."""
    d, s = 4, 32
    q = np.array([2.0, 0.0, 0.0, 0.0])
    k = np.zeros((64, d))
    k[32:64] = [3.0, 1.0, 0.0, 0.0]
    prm = Params(lam=0.0)
    r, _ = oracle.fsb_rerank_score(q, k, 0.0, 100, 1, prm)
    assert r == pytest.approx(3.0 + np.log(s), rel=1e-14)  # q . k / sqrt(4) = 3
    k2 = np.zeros((64, d))
    k2[32:48] = [1000.0, 0, 0, 0]
    k2[48:64] = [999.0, 0, 0, 0]
    r2, _ = oracle.fsb_rerank_score(q, k2, 0.0, 100, 1, prm)
    assert r2 == pytest.approx(np.log(16.0) + 999.0 + np.log(np.exp(1.0) + 1.0), rel=1e-14)


# ------------------------------------------------------------ whole branch ----

def test_first_block_empty_and_causal():
    """The first block has no long-range cells (zero output); later keys and values never
    change earlier outputs (each block sees cells completed before its start)."""
    N, d = 1024, 8
    q, k, v = data(11, N, d)
    fb = FsbParams(tau=1.0, Wb=4)
    r1 = oracle.fsb_head(q, k, v, prm=Params(), fb=fb)
    assert np.all(r1["sel"][:128] == -1) and np.all(r1["out"][:128] == 0)
    k2, v2 = k.copy(), v.copy()
    k2[600:] = 5.0 * rng(12).normal(size=(N - 600, d))
    v2[600:] = rng(13).normal(size=(N - 600, d))
    r2 = oracle.fsb_head(q, k2, v2, prm=Params(), fb=fb)
    blk = 600 // 128  # queries of blocks starting at or before 600 - 32 see none of the change
    np.testing.assert_array_equal(r1["sel"][: blk * 128 + 128], r2["sel"][: blk * 128 + 128])
    np.testing.assert_array_equal(r1["out"][: blk * 128 + 128], r2["out"][: blk * 128 + 128])


def test_selection_is_top_k_of_candidates_and_readout():
    """S_i = the K best candidates by Eq. 12 (ties to the smaller id), read with Eq. 9 and
    Eq. 17: checked against the reranked scores of B_i one by one."""
    N, d = 1536, 8
    q, k, v = data(14, N, d)
    fb = FsbParams(tau=2.0, Wb=3)
    prm = Params(K=3)
    res = oracle.fsb_head(q, k, v, prm=prm, fb=fb)
    kbar, a = res["kbar"], res["a"]
    for i in range(128, N, 37):
        cand = [c for c in res["cand"][i] if c >= 0]
        assert len(cand) <= 2 * fb.Wb
        sc = {c: oracle.fsb_rerank_score(q[i], k, a[c], i, c, prm)[0] for c in cand}
        expect = sorted(cand, key=lambda c: (-sc[c], c))[: prm.K]
        assert list(res["sel"][i][: len(expect)]) == expect
        np.testing.assert_allclose(res["out"][i], oracle.readout(q[i], k, v, expect, None, prm), rtol=0, atol=0)
