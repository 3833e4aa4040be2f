"""Pins of the fp64 oracle against what the FreeSolo page and mathematics fix.

None of these tests re-types the oracle's formulas: each checks a closed form,
a value printed on the page, an invariant the page states, or a brute-force
recount on a tiny input.  Page: "FreeSolo: Linear-time Sparse Attention with
Zero-Shot Length Extrapolation" (arXiv 2610.17191).
"""

import numpy as np
import pytest

import oracle
from oracle import Params

# Textbook constants (Abramowitz & Stegun, Table 7.1), not computed by any routine here.
ERF_1 = 0.8427007929497148693
ERF_2 = 0.9953222650189527342
ERFC_2 = 0.0046777349810472658


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- Eq. 5 ----

def test_keypoint_cell_closed_form(golden):
    """App. D.2 'A keypoint can mark a cell': one nonzero key k* gives kbar = k*/s, a = ||k*||."""
    s = golden["hyperparameters"]["s"]
    d = 16
    k = np.zeros((4 * s, d))
    kstar = rng(0).normal(size=d) * 3.0
    k[2 * s + 7] = kstar
    kbar, a = oracle.cell_summaries(k, Params(s=s))
    np.testing.assert_allclose(kbar[2], kstar / s, rtol=0, atol=1e-15)
    assert a[2] == pytest.approx(float(np.sqrt(np.sum(kstar ** 2))), rel=1e-15)
    assert np.all(kbar[[0, 1, 3]] == 0) and np.all(a[[0, 1, 3]] == 0)


def test_constant_and_ramp_keys_closed_form():
    """Constant keys: kbar = u, a = ||u||.  Ramp k_j = j e: kbar_c = (cs + (s-1)/2) e, a_c = ((c+1)s-1)||e||."""
    s, d = 8, 5
    u = np.array([1.0, -2.0, 0.5, 3.0, 0.25])
    kbar, a = oracle.cell_summaries(np.tile(u, (3 * s + 5, 1)), Params(s=s))
    assert kbar.shape == (3, d)  # the trailing partial cell has no summary
    np.testing.assert_allclose(kbar, np.tile(u, (3, 1)), atol=1e-14)
    np.testing.assert_allclose(a, np.full(3, np.sqrt(14.3125)), rtol=1e-15)
    e = np.array([0.5, 0.0, -1.0, 2.0, 1.0])
    N = 6 * s
    ramp = np.arange(N)[:, None] * e[None, :]
    kbar, a = oracle.cell_summaries(ramp, Params(s=s))
    for c in range(6):
        np.testing.assert_allclose(kbar[c], (c * s + (s - 1) / 2) * e, atol=1e-12)
        assert a[c] == pytest.approx(((c + 1) * s - 1) * 2.5, rel=1e-14)  # ||e|| = 2.5


def test_cell_centre_worked_example(golden):
    """App. D.2: cell 2981 is centred at 95,408, and the final query of a 262,010-token
    input is 166,601 tokens from that centre.  With q = 0 and a = 1 the score is the
    prior alone; choosing 2 sigma = 166,601 makes it erf(1) exactly when p_c is right."""
    ex = golden["needle_cell"]
    s = golden["hyperparameters"]["s"]
    assert (ex["cell"] + 0.5) * s == ex["centre"]
    i_final = ex["input_tokens"] - 1  # zero-based position of the final prompt query
    assert i_final - ex["centre"] == ex["final_query_distance"]
    prm = Params(s=s, sigma=ex["final_query_distance"] / 2.0, lam=1.0)
    r = oracle.cell_score(np.zeros(8), np.ones(8), 1.0, i_final, ex["cell"], prm)
    assert r == pytest.approx(ERF_1, abs=1e-14)
    # the neighbouring cells would be 32 tokens off: the score must move
    r_next = oracle.cell_score(np.zeros(8), np.ones(8), 1.0, i_final, ex["cell"] + 1, prm)
    assert abs(r_next - ERF_1) > 1e-5


def test_prior_at_minimal_offset_is_erf2(golden):
    """Sec. 5 / App. D.1: at s=32 and sigma=4 the smallest eligible offset i - p_c = s/2
    gives g_h = erf(2) ~ 0.9953.  Also fixes the argument as Delta/(2 sigma) and the sign."""
    hp = golden["hyperparameters"]
    prm = Params(s=hp["s"], sigma=hp["sigma"], lam=2.0)
    # query at the first position of block 1 (b_i = 128); last available cell c = 3, p_c = 112
    r = oracle.cell_score(np.zeros(4), np.zeros(4), 3.0, 128, 3, prm)
    assert r == pytest.approx(6.0 * ERF_2, abs=1e-13)
    assert round(r / 6.0, golden["erf_2"]["printed_digits"]) == golden["erf_2"]["value"]
    # a cell one block further back is saturated: erf(10) == 1 to fp64
    r_far = oracle.cell_score(np.zeros(4), np.zeros(4), 3.0, 128 + 64, 3, prm)
    assert r_far == pytest.approx(6.0, abs=1e-12)


def test_content_term_scale():
    """Eq. 7 with lambda = 0: r = q . kbar / sqrt(d), using the head dimension d."""
    d = 64
    q = np.zeros(d); q[3] = 2.0; q[10] = -1.0
    kb = np.zeros(d); kb[3] = 5.0; kb[10] = 4.0; kb[11] = 100.0
    r = oracle.cell_score(q, kb, 7.0, 1000, 2, Params(lam=0.0))
    assert r == pytest.approx((10.0 - 4.0) / 8.0, abs=1e-15)


# ---------------------------------------------------------------- Eq. 6 ----

def test_availability_counts(golden):
    """Eq. 6: |C_i| = number of cells ending at or before the block start."""
    hp = golden["hyperparameters"]
    s, B = hp["s"], hp["B"]
    assert oracle.available_count(0, s) == 0  # "the first block has no long-range cells"
    assert oracle.available_count(B, s) == golden["cells_per_block"]["value"]
    ex = golden["eligible_cells_at_4096"]
    last_block_start = B * ((ex["N"] - 1) // B)
    assert oracle.available_count(last_block_start, s) == ex["last_block_eligible_cells"]
    assert ex["last_block_eligible_cells"] > ex["P_plus_W"] == hp["P"] + hp["W"]


def test_full_head_block_structure(golden):
    """Whole-head run: block 0 empty and zero, FS prefixes grow by 4 cells per block,
    and the 4096-token last block has 124 eligible cells but at most P+W retained."""
    ex = golden["eligible_cells_at_4096"]
    N, d = ex["N"], 8
    g = rng(1)
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    fs = oracle.head(q, k, v, prm=Params(prune=False), want_out=True)
    assert np.all(fs["sel"][:128] == -1) and np.all(fs["out"][:128] == 0)
    assert list(fs["n_ret"][:5]) == [0, 4, 8, 12, 16]
    assert fs["n_ret"][-1] == ex["last_block_eligible_cells"]
    fsl = oracle.head(q, k, v, prm=Params(prune=True), want_out=False)
    assert fsl["n_ret"][-1] <= ex["P_plus_W"]
    assert fsl["n_ret"][-1] >= 64


# ---------------------------------------------------------------- Eq. 8 ----

def _brute_retained(a, n_avail, P, W):
    """Rank-count formulation: c is in TopP iff fewer than P cells of C outrank it."""
    keep = set()
    for c in range(n_avail):
        outrank = sum(1 for x in range(n_avail) if a[x] > a[c] or (a[x] == a[c] and x < c))
        if outrank < P:
            keep.add(c)
    keep |= set(range(max(0, n_avail - W), n_avail))
    return sorted(keep)


@pytest.mark.parametrize("P,W", [(0, 0), (0, 3), (3, 0), (4, 2), (7, 5), (64, 8)])
def test_retention_brute_force(P, W):
    g = rng(P * 10 + W)
    for trial in range(30):
        n = int(g.integers(0, 40))
        a = np.round(g.uniform(0, 4, size=max(n, 1)), 0 if trial % 2 else 3)  # forces ties half the time
        ids, _ = oracle.retained(a, n, Params(P=P, W=W, prune=True))
        assert list(ids) == _brute_retained(a, n, P, W)
        assert len(ids) <= P + W
        if n <= P:
            assert list(ids) == list(range(n))  # A == C when the prefix fits in P


def test_retention_invariants():
    """|A| in [min(P,|C|), P+W]; Recent subset of A; every retained non-recent cell
    outranks every discarded cell by (a desc, id asc) (App. D.3)."""
    g = rng(7)
    P, W = 10, 4
    for _ in range(50):
        n = int(g.integers(0, 60))
        a = g.lognormal(size=max(n, 1))
        ids, _ = oracle.retained(a, n, Params(P=P, W=W))
        S = set(ids.tolist())
        assert min(P, n) <= len(S) <= P + W
        assert set(range(max(0, n - W), n)) <= S
        kept = [c for c in S if c < n - W]
        dropped = [c for c in range(n) if c not in S]
        for c in kept:
            for x in dropped:
                assert a[c] > a[x] or (a[c] == a[x] and c < x)


def test_incremental_topp_eq15():
    """App. C Eq. 15: TopP(C u D) = TopP(TopP(C) u D) with the common tie rule.  A Python
    merge that only ever sees the previous top-P plus 4 new cells must reproduce the
    oracle's per-block retained sets (which sort the full prefix every block)."""
    g = rng(11)
    P, W, s, B = 6, 3, 4, 16
    N, d = 40 * B, 3
    k = g.normal(size=(N, d)) * g.lognormal(size=(N, 1))
    k[::37] *= 4.0
    k = np.round(k, 1)  # coarse keys so that norms tie now and then
    prm = Params(s=s, B=B, P=P, W=W, K=2)
    res = oracle.head(np.zeros((N, d)), k, np.zeros((N, d)), prm=prm, want_out=False)
    a = res["a"]
    top = []  # list of (a, id) in (a desc, id asc) order
    for blk in range(N // B):
        n_avail = blk * B // s
        if blk > 0:
            new = list(range(n_avail - B // s, n_avail))
            top = sorted(top + [(a[c], c) for c in new], key=lambda t: (-t[0], t[1]))[:P]
        expect = sorted(set(c for _, c in top) | set(range(max(0, n_avail - W), n_avail)))
        got = res["retained"][blk][: res["n_ret"][blk]]
        assert list(got) == expect, blk


def test_gap_p_known_boundary():
    """gap_P is the relative gap |a_(P) - a_(P+1)| / max(|a_(P)|, |a_(P+1)|) between the P-th
    and (P+1)-th largest key norms of the prefix (near-ties there decide which cell Eq. 8
    keeps).  Hand-built norms with known gaps at every rank; +inf when there is no boundary."""
    a = np.array([3.0, 10.0, 7.5, 9.0, 1.0, 8.0, 6.0])  # sorted: 10, 9, 8, 7.5, 6, 3, 1
    srt = sorted(a, reverse=True)
    for P in range(1, len(a)):
        _, gap = oracle.retained(a, len(a), Params(P=P, W=0))
        expect = (srt[P - 1] - srt[P]) / srt[P - 1]
        assert gap == pytest.approx(expect, rel=1e-15), P
    assert oracle.retained(a, len(a), Params(P=len(a), W=0))[1] == np.inf  # the whole prefix fits
    assert oracle.retained(a, 4, Params(P=5, W=0))[1] == np.inf             # only the first 4 cells available
    assert oracle.retained(a, len(a), Params(P=0, W=2))[1] == np.inf        # no TopP at all
    # only the available prefix counts: cells 0..3 are 3, 10, 7.5, 9 -> P=2 boundary is 9 vs 7.5
    assert oracle.retained(a, 4, Params(P=2, W=0))[1] == pytest.approx(1.5 / 9.0, rel=1e-15)
    # an exact tie at the boundary has gap 0 (and the smaller id wins, App. C)
    ids, gap = oracle.retained(np.array([5.0, 2.0, 5.0, 1.0]), 4, Params(P=1, W=0))
    assert gap == 0.0 and list(ids) == [0]
    # the per-block gap reported by the whole-head run is the same quantity
    g = rng(18)
    N, d = 2048, 4
    k = g.normal(size=(N, d)) * g.lognormal(size=(N, 1))
    prm = Params(P=5, W=2)
    res = oracle.head(np.zeros((N, d)), k, np.zeros((N, d)), prm=prm, want_out=False)
    for blk in range(1, N // 128):
        n = blk * 4
        srt = np.sort(res["a"][:n])[::-1]
        expect = (srt[4] - srt[5]) / srt[4] if n > 5 else np.inf
        assert res["gap_p"][blk] == pytest.approx(expect, rel=1e-14)


# ---------------------------------------------------------- selection ------

def test_topk_rank_count_and_gap():
    """T_i holds exactly the cells outranked (score desc, id asc) by fewer than K others."""
    g = rng(3)
    s, B, N, d = 4, 16, 16 * 12, 6
    prm = Params(s=s, B=B, P=5, W=2, K=3)
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    res = oracle.head(q, k, v, prm=prm, want_scores=True)
    for i in range(N):
        blk = i // B
        A = res["retained"][blk][: res["n_ret"][blk]]
        r = res["scores"][i][: len(A)]
        chosen = []
        for x, c in enumerate(A):
            outrank = sum(1 for y in range(len(A)) if r[y] > r[x] or (r[y] == r[x] and A[y] < c))
            if outrank < prm.K:
                chosen.append((outrank, c))
        expect = [c for _, c in sorted(chosen)] + [-1] * (prm.K - len(chosen))
        assert list(res["sel"][i]) == expect
        if len(A) > prm.K:  # measured against the term sizes, which are at least the scores
            rs = np.sort(r)[::-1]
            plain = abs(rs[prm.K - 1] - rs[prm.K]) / max(abs(rs[prm.K - 1]), abs(rs[prm.K]))
            assert 0 <= res["gap_k"][i] <= plain * (1 + 1e-12)


def test_gap_k_against_term_sizes_closed_form():
    """The K/K+1 gap is taken relative to the size of the terms Eq. 7 sums,
    sum_f |q_f kbar_f| / sqrt(d) + lambda a_c |g|, not to the scores themselves (content
    terms can cancel; fp32 scores are exact only to roundings of that size).  s = 1 makes
    kbar_c = k_c and a_c = |k_c|; a vanishing sigma makes g = 1 for every earlier cell."""
    d, s, B = 2, 1, 4
    k = np.array([[3.0, -2.0], [0.5, 0.4], [-1.0, -1.0], [0.1, 0.0], [0.0, 0.0], [0.0, 0.0], [0.0, 0.0],
                  [0.0, 0.0]])
    q = np.tile([1.0, 1.0], (len(k), 1))
    # query 4 (block 1) sees cells 0..3 with content scores 1, 0.9, -2, 0.1 (times 1/sqrt 2)
    res = oracle.head(q, k, np.zeros_like(k), prm=Params(s=s, B=B, K=1, prune=False, lam=0.0), want_out=False)
    assert res["sel"][4][0] == 0
    assert res["gap_k"][4] == pytest.approx(0.1 / 5.0, rel=1e-14)   # |1 - 0.9| / max(5, 0.9)
    prm = Params(s=s, B=B, K=1, prune=False, lam=0.5, sigma=1e-9)
    res = oracle.head(q, k, np.zeros_like(k), prm=prm, want_out=False)
    r = [(1.0 + 0.5 * np.sqrt(13.0) * np.sqrt(2)) / np.sqrt(2), (0.9 + 0.5 * np.sqrt(0.41) * np.sqrt(2)) / np.sqrt(2)]
    m = [(5.0 + 0.5 * np.sqrt(13.0) * np.sqrt(2)) / np.sqrt(2), (0.9 + 0.5 * np.sqrt(0.41) * np.sqrt(2)) / np.sqrt(2)]
    assert oracle.cell_score(q[4], k[0], np.sqrt(13.0), 4, 0, prm) == pytest.approx(r[0], rel=1e-14)
    assert oracle.cell_score_mag(q[4], k[0], np.sqrt(13.0), 4, 0, prm) == pytest.approx(m[0], rel=1e-14)
    assert oracle.cell_score_mag(q[4], k[2], np.sqrt(2.0), 4, 2, prm) == pytest.approx(
        (2.0 + 0.5 * np.sqrt(2.0) * np.sqrt(2)) / np.sqrt(2), rel=1e-14)          # |-1| + |-1|, no cancellation
    # cell 2 scores (-2 + 1) / sqrt 2 < cell 1's; the boundary pair is cells 0 and 1
    assert res["gap_k"][4] == pytest.approx((r[0] - r[1]) / max(m), rel=1e-13)
    # with K = 2 the pair that decides the order of the two selected cells counts too:
    # content scores 1, 0.9, 0.1 (sizes 5, 0.9, 0.1): min(0.1 / 5, 0.8 / 0.9) = 0.02, not the
    # boundary's 0.889
    res2 = oracle.head(q, k, np.zeros_like(k), prm=Params(s=s, B=B, K=2, prune=False, lam=0.0), want_out=False)
    assert list(res2["sel"][4]) == [0, 1]
    assert res2["gap_k"][4] == pytest.approx(0.1 / 5.0, rel=1e-14)


# ------------------------------------------------------------ readout ------

def _rmsnorm(u, g, eps):
    return g * u / np.sqrt(np.mean(u * u) + eps)


def test_dense_attention_when_K_covers_prefix():
    """With FS (A = C) and K >= |A_i|, S_i is every token before the block start, so the
    branch is dense softmax attention over j < b_i followed by RMSNorm (brute force)."""
    g = rng(5)
    s, B, N, d = 8, 32, 32 * 6, 8
    prm = Params(s=s, B=B, K=64, prune=False, eps=1e-8)
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    gain = g.uniform(0.5, 1.5, size=d)
    res = oracle.head(q, k, v, gain, prm=prm)
    for i in range(N):
        b_i = B * (i // B)
        if b_i == 0:
            assert np.all(res["out"][i] == 0)
            continue
        logits = k[:b_i] @ q[i] / np.sqrt(d)
        w = np.exp(logits - logits.max()); w /= w.sum()
        np.testing.assert_allclose(res["out"][i], _rmsnorm(w @ v[:b_i], gain, 1e-8), rtol=1e-11, atol=1e-12)


def test_masked_dense_attention_with_pruning():
    """FS-L with K >= |A_i|: dense softmax over the tokens of the retained cells only."""
    g = rng(6)
    s, B, N, d = 8, 32, 32 * 10, 8
    prm = Params(s=s, B=B, P=5, W=3, K=16, prune=True)
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    k *= g.lognormal(size=(N, 1))
    res = oracle.head(q, k, v, prm=prm)
    for i in range(B, N):
        blk = i // B
        A = res["retained"][blk][: res["n_ret"][blk]]
        toks = np.concatenate([np.arange(c * s, (c + 1) * s) for c in A])
        logits = k[toks] @ q[i] / np.sqrt(d)
        w = np.exp(logits - logits.max()); w /= w.sum()
        np.testing.assert_allclose(res["out"][i], _rmsnorm(w @ v[toks], 1.0, prm.eps), rtol=1e-11, atol=1e-12)


def test_empty_selection_is_zero():
    """Eq. 9: both outputs are zero when S_i is empty (here P = W = 0 empties every A_i)."""
    g = rng(8)
    N, d = 512, 8
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    res = oracle.head(q, k, v, prm=Params(P=0, W=0))
    assert np.all(res["sel"] == -1) and np.all(res["out"] == 0) and np.all(res["n_ret"] == 0)


def test_zero_query_reads_mean_value():
    """q = 0 makes every logit 0: u is the plain mean of the selected values (closed form),
    and the selection is by the prior alone, i.e. by a_c erf(...)."""
    g = rng(9)
    N, d = 1024, 16
    k = g.normal(size=(N, d)) * g.lognormal(size=(N, 1))
    v = g.normal(size=(N, d))
    gain = g.uniform(0.5, 1.5, size=d)
    res = oracle.head(np.zeros((N, d)), k, v, gain, prm=Params())
    for i in range(128, N, 37):
        toks = np.concatenate([np.arange(c * 32, (c + 1) * 32) for c in res["sel"][i] if c >= 0])
        np.testing.assert_allclose(res["out"][i], _rmsnorm(v[toks].mean(0), gain, 1e-8), rtol=1e-12, atol=1e-13)


def test_readout_of_given_selection():
    """Eq. 9 + Eq. 17 for a caller-given selection (the check of near-tie queries reads out
    the GPU's own choice with it): brute-force softmax over exactly the listed cells' tokens,
    -1 entries ignored, an empty selection gives 0, q = 0 gives the mean of the values."""
    g = rng(19)
    s, N, d = 32, 512, 8
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    gain = g.uniform(0.5, 1.5, size=d)
    prm = Params()
    for cells in ([3], [0, 7, 2], [9, -1, 4, -1], [5, 1, 14, 6]):
        toks = np.concatenate([np.arange(c * s, (c + 1) * s) for c in cells if c >= 0])
        logits = k[toks] @ q[300] / np.sqrt(d)
        w = np.exp(logits - logits.max()); w /= w.sum()
        np.testing.assert_allclose(oracle.readout(q[300], k, v, cells, gain, prm),
                                   _rmsnorm(w @ v[toks], gain, prm.eps), rtol=1e-12, atol=1e-13)
    assert np.all(oracle.readout(q[300], k, v, [-1, -1], gain, prm) == 0)
    toks = np.concatenate([np.arange(c * s, (c + 1) * s) for c in (2, 11)])
    np.testing.assert_allclose(oracle.readout(np.zeros(d), k, v, [11, 2], None, prm),
                               _rmsnorm(v[toks].mean(0), 1.0, prm.eps), rtol=1e-12, atol=1e-13)


def test_rmsnorm_epsilon_placement(golden):
    """Eq. 17: eps sits inside the root, added to the mean square.  With values so small
    that ||u||^2/d << eps the output is g u / sqrt(eps); with large values eps is negligible."""
    eps = golden["rmsnorm_eps"]["value"]
    g = rng(10)
    N, d = 256, 8
    k = g.normal(size=(N, d))
    v = np.full((N, d), 1e-7)  # every selected value equals 1e-7 -> u = 1e-7 exactly
    res = oracle.head(np.zeros((N, d)), k, v, prm=Params(eps=eps))
    i = 200
    expect = 1e-7 / np.sqrt(1e-14 + eps)
    np.testing.assert_allclose(res["out"][i], np.full(d, expect), rtol=1e-12)
    assert expect < 1.0  # would be exactly 1 if eps were dropped


def test_value_scale_invariance():
    """App. D.2: when ||u||^2/d >> eps, RMSNorm cancels the amplitude, so o(alpha v) = o(v)."""
    g = rng(12)
    N, d = 640, 16
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    r1 = oracle.head(q, k, v)
    r2 = oracle.head(q, k, 7.5 * v)
    # the residual is O(eps / mean(u^2)) ~ 1e-6; without RMSNorm it would be a factor 7.5
    np.testing.assert_allclose(r1["out"], r2["out"], rtol=1e-4, atol=1e-5)


def test_translation_by_one_block():
    """App. D.1 'Position dependence': shifting tokens, cells, blocks and boundaries by B
    leaves the operator unchanged.  Prepend B tokens with zero key and value: their cells
    have a = 0 and score exactly 0, so they are never chosen over the (positive-score)
    original cells, every prior offset i - p_c is unchanged, and cell ids shift by B/s."""
    g = rng(13)
    N, d, B, s = 1024, 16, 128, 32
    q = g.normal(size=(N, d))
    k = g.normal(size=(N, d)) * g.lognormal(size=(N, 1)) * 2.0
    v = g.normal(size=(N, d))
    pad = np.zeros((B, d))
    base = oracle.head(q, k, v, want_scores=True)
    shifted = oracle.head(np.vstack([g.normal(size=(B, d)), q]), np.vstack([pad, k]), np.vstack([pad, v]))
    assert np.nanmin(base["scores"]) > 0
    np.testing.assert_allclose(shifted["out"][B:], base["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(shifted["sel"][2 * B:], base["sel"][B:] + B // s)


def test_saturated_prior_bound_eq16(golden):
    """App. D.1 Eq. 16: 0 <= r_inf - r <= lambda a_c erfc(s/(4 sigma)), with erfc(2) ~ 0.004678
    at s=32, sigma=4; r_inf is the constant-gate score (a vanishing sigma gives g = 1)."""
    g = rng(14)
    N, d = 2048, 16
    q = g.normal(size=(N, d))
    k = g.normal(size=(N, d)) * g.lognormal(sigma=0.5, size=(N, 1))
    v = g.normal(size=(N, d))
    lam = 1.0
    r = oracle.head(q, k, v, prm=Params(lam=lam), want_scores=True)
    rinf = oracle.head(q, k, v, prm=Params(lam=lam, sigma=1e-12), want_scores=True)
    assert round(ERFC_2, 6) == golden["erfc_2"]["value"]
    diff = rinf["scores"] - r["scores"]
    for i in range(128, N):
        blk = i // 128
        A = r["retained"][blk][: r["n_ret"][blk]]
        dd = diff[i][: len(A)]
        assert np.all(dd >= -1e-12)
        assert np.all(dd <= lam * r["a"][A] * ERFC_2 + 1e-12)


def test_constant_gate_stability_criterion():
    """App. D.1: if the K-th/(K+1)-th gap of the constant-gate scores exceeds
    delta_max = max_c lambda a_c erfc((i-p_c)/(2 sigma)), the selection is unchanged."""
    g = rng(15)
    N, d = 2048, 16
    q = g.normal(size=(N, d)) * 3.0
    k = g.normal(size=(N, d)) * g.lognormal(sigma=0.5, size=(N, 1))
    v = g.normal(size=(N, d))
    r = oracle.head(q, k, v, want_scores=True)
    rinf = oracle.head(q, k, v, prm=Params(sigma=1e-12), want_scores=True)
    checked = 0
    for i in range(128, N):
        blk = i // 128
        n = r["n_ret"][blk]
        if n <= 4:
            continue
        ri = np.sort(rinf["scores"][i][:n])[::-1]
        delta_max = np.max(rinf["scores"][i][:n] - r["scores"][i][:n])
        if ri[3] - ri[4] > delta_max:
            assert set(r["sel"][i]) == set(rinf["sel"][i])
            checked += 1
    assert checked > 100


def test_fsl_equals_fs_when_prefix_fits_in_P():
    """FS-L and FS coincide while |C_i| <= P (every available cell is in TopP): the
    1024-token, 32-cell workload never has more than 28 available cells."""
    g = rng(16)
    N, d = 1024, 16
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    k *= g.lognormal(sigma=0.5, size=(N, 1))
    a = oracle.head(q, k, v, prm=Params(prune=True))
    b = oracle.head(q, k, v, prm=Params(prune=False))
    np.testing.assert_array_equal(a["sel"], b["sel"])
    np.testing.assert_array_equal(a["out"], b["out"])
    assert a["n_ret"].max() == 28


def test_partial_range_matches_full_run():
    """Evaluating a sub-range of queries gives the same rows as the full run."""
    g = rng(17)
    N, d = 1000, 8
    q, k, v = (g.normal(size=(N, d)) for _ in range(3))
    full = oracle.head(q, k, v)
    part = oracle.head(q, k, v, i_lo=300, i_hi=777)
    np.testing.assert_array_equal(part["sel"], full["sel"][300:777])
    np.testing.assert_array_equal(part["out"], full["out"][300:777])


# ------------------------------------------- local branch (Eqs. 3-4) and Eq. 2 ----

def test_local_window_zero_reads_own_value():
    """Sec. 3.2 with w = 0: L_i = {i}, so the local output is v_i whatever q and k are."""
    r = rng(40)
    q, k, v = (r.normal(size=(50, 8)) for _ in range(3))
    np.testing.assert_allclose(oracle.local(q, k, v, w=0), v, rtol=0, atol=1e-15)


def test_local_zero_query_reads_window_mean():
    """q = 0 makes every logit equal, so o_i is the mean of v over [max(0, i - w), i]:
    a full window holds w + 1 tokens (Sec. 3.2)."""
    r = rng(41)
    N, d, w = 60, 6, 7
    k, v = r.normal(size=(N, d)), r.normal(size=(N, d))
    o = oracle.local(np.zeros((N, d)), k, v, w=w)
    for i in range(N):
        np.testing.assert_allclose(o[i], v[max(0, i - w): i + 1].mean(axis=0), rtol=0, atol=1e-14)


def _softmax_read(logits, vals):
    p = np.exp(logits - logits.max())
    return (p / p.sum()) @ vals


def test_local_rope_angle_difference_closed_form():
    """d = 2 has one pair with theta_0 = 1.  For q = (1, 0) and k = (0, 1) the rotated
    product is cos(i)(-sin j) + sin(i)cos(j) = sin(i - j) (angle difference), so the
    logits are sin(i - j) / sqrt(2) (Eq. 3)."""
    N, w = 40, 9
    q = np.tile([1.0, 0.0], (N, 1))
    k = np.tile([0.0, 1.0], (N, 1))
    v = rng(42).normal(size=(N, 2))
    o = oracle.local(q, k, v, w=w)
    for i in range(N):
        js = np.arange(max(0, i - w), i + 1)
        np.testing.assert_allclose(o[i], _softmax_read(np.sin(i - js) / np.sqrt(2.0), v[js]), rtol=0, atol=1e-13)


def test_local_rope_frequency_closed_form():
    """theta_m = base^(-2m/d): with d = 4 and base 100, pair 1 turns by 100^(-1/2) = 0.1
    rad per position, so q = (0, 0, 1, 0), k = (0, 0, 0, 1) give sin(0.1 (i - j)) / 2."""
    N, w = 30, 12
    q = np.tile([0.0, 0.0, 1.0, 0.0], (N, 1))
    k = np.tile([0.0, 0.0, 0.0, 1.0], (N, 1))
    v = rng(43).normal(size=(N, 4))
    o = oracle.local(q, k, v, w=w, rope_base=100.0)
    for i in range(N):
        js = np.arange(max(0, i - w), i + 1)
        np.testing.assert_allclose(o[i], _softmax_read(np.sin(0.1 * (i - js)) / 2.0, v[js]), rtol=0, atol=1e-13)


def test_local_relative_position_invariance():
    """Eq. 3: the logits depend on j - i only, so prepending m tokens leaves the output
    of every query whose window holds none of them unchanged."""
    r = rng(44)
    N, d, w, m = 80, 8, 10, 13
    q, k, v = (r.normal(size=(N, d)) for _ in range(3))
    pre = [r.normal(size=(m, d)) for _ in range(3)]
    o = oracle.local(q, k, v, w=w)
    o2 = oracle.local(np.vstack([pre[0], q]), np.vstack([pre[1], k]), np.vstack([pre[2], v]), w=w)
    np.testing.assert_allclose(o2[m + w:], o[w:], rtol=0, atol=1e-12)


def test_local_relative_form_brute_force():
    """Tiny brute force through Eq. 3's second form, q_i^T R(j - i) k_j, with R built as an
    explicit block-diagonal rotation matrix (the oracle rotates q and k separately)."""
    r = rng(45)
    N, d, w, base = 25, 8, 6, 10000.0
    q, k, v = (r.normal(size=(N, d)) for _ in range(3))

    def rot(p):
        R = np.zeros((d, d))
        for mm in range(d // 2):
            a = p * base ** (-2.0 * mm / d)
            R[2 * mm:2 * mm + 2, 2 * mm:2 * mm + 2] = [[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]]
        return R

    o = oracle.local(q, k, v, w=w, rope_base=base)
    for i in range(N):
        js = np.arange(max(0, i - w), i + 1)
        logits = np.array([q[i] @ rot(j - i) @ k[j] for j in js]) / np.sqrt(d)
        np.testing.assert_allclose(o[i], _softmax_read(logits, v[js]), rtol=0, atol=1e-12)


def test_local_branch_combination_eq2():
    """Eq. 2: o = o_sr + alpha_h o_lr.  With alpha = 0 the local branch alone; the
    difference between two alphas is their difference times the long-range output."""
    r = rng(46)
    N, d, w = 30, 4, 5
    q, k, v, olr = (r.normal(size=(N, d)) for _ in range(4))
    o0 = oracle.local(q, k, v, w=w)
    np.testing.assert_array_equal(oracle.local(q, k, v, w=w, alpha=0.0, o_lr=olr), o0)
    o1 = oracle.local(q, k, v, w=w, alpha=1.25, o_lr=olr)
    np.testing.assert_allclose(o1 - o0, 1.25 * olr, rtol=0, atol=1e-14)
