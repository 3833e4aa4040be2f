"""Shared helpers of the GPU parity tests: seeded inputs on both sides, the oracle
on (sequence, head) samples, and the comparison rules.

Comparison rules (written once, used by every parity test):
  * cell ids (retained sets, selections) are compared exactly, except where the
    oracle reports a near-tie: a gap below 1e-6 between the K-th and (K+1)-th
    routing scores of a query, relative to the size of the terms each score is
    summed from (the content term can cancel: a score of 0.3 may be the sum of
    terms of size 3, and any fp32 evaluation is exact only to roundings of that
    size), or a relative gap below 1e-6 between the P-th and (P+1)-th key norms
    of a block's prefix.  Several selections are then correct, so such a
    query is not compared with the oracle's choice but validated: the GPU's
    cells must be distinct cells the query can reach, a top-K of the oracle's
    own fp64 scores within the 1e-6 band and listed in that order, and the
    GPU's output must match the oracle's readout of the GPU's own selection.
    Every query is checked one way or the other; near-ties are counted.
  * outputs: fp32 tensors, per row max|o - o_ref| <= 1e-5 * max(1, max|o_ref|);
    bf16 tensors, elementwise |o - o_ref| <= 2e-2.  Rows the oracle leaves
    exactly zero (no selected cell) must be exactly zero.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

NEAR_TIE = 1e-6
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# Readout backward bar: |gpu - oracle| <= BWD_REL[dtype] x the oracle's first-order error
# scale + BWD_FLOOR x the tensor's largest scale.  The scale is a worst-case first-order
# bound, so the bar is the relative rounding e of the path's arithmetic itself: for bf16
# tensors the split products (p du, du v, dS k, ...) keep each factor to 2^-17, two factors
# per product: e = 2^-16; for fp32 tensors the products are fp32 and the largest error is in
# the softmax exponent, about 2^-23 |lse| with |lse| < 2^5: e = 2^-19 (relative, in p).
BWD_REL = {"bf16": 2.0 ** -16, "f32": 2.0 ** -19}
BWD_FLOOR = 1e-7


def bwd_beyond_bar(got, ref, scale, dtype):
    """Elements of a backward result beyond the bar (see BWD_REL)."""
    import numpy as np
    bound = BWD_REL[dtype] * scale + BWD_FLOOR * (scale.max() if scale.size else 0.0)
    return np.abs(np.asarray(got, dtype=np.float64) - ref) > bound


def inputs(w: synth.Workload):
    return {x: synth.tensor(w, x) for x in "qkv"}


def oracle_params(p, sigma=4.0, lam=1.0) -> oracle.Params:
    return oracle.Params(s=p.s, B=p.B, P=p.P, W=p.W, K=p.K, prune=p.prune, sigma=sigma, lam=lam, eps=p.eps)


def run_oracle(w, host, p, heads, sigma=4.0, lam=1.0, gain=None, i_lo=0, i_hi=None):
    """Oracle results per sampled (b, h) pair (inputs widened exactly to fp64).  Each
    result also carries its fp64 inputs and parameters, which the near-tie
    validation of compare_head needs."""
    def one(bh):
        b, h = bh
        op = oracle_params(p, sigma[h] if isinstance(sigma, (list, tuple)) else sigma,
                           lam[h] if isinstance(lam, (list, tuple)) else lam)
        g = None if gain is None else gain[h]
        x = tuple(synth.to_f64(host[t][b, h], w.dtype) for t in "qkv")
        ref = oracle.head(*x, g, op, i_lo, i_hi)
        ref["inputs"] = x + (g,)
        ref["prm"] = op
        return bh, ref

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return dict(ex.map(one, heads))


def excluded_queries(ref, p, i_lo, n):
    """Queries whose selection is decided by a near-tie (see module docstring)."""
    gap_k = ref["gap_k"]
    blocks = (np.arange(i_lo, i_lo + n) // p.B)
    gap_p = ref["gap_p"][blocks]
    return (gap_k < NEAR_TIE) | (np.nan_to_num(gap_p, nan=np.inf) < NEAR_TIE)


def rel_gap(x, y):
    m = max(abs(x), abs(y))
    return abs(x - y) / m if m > 0 else 0.0


def boundary_pool(a, n_avail, P, band=NEAR_TIE):
    """Cells of the prefix [0, n_avail) whose key norm lies within the near-tie band of
    the P-th / (P+1)-th largest norms: the cells a near-tie at the TopP boundary may
    swap (empty when that boundary is not a near-tie)."""
    if P <= 0 or n_avail <= P:
        return set()
    srt = np.sort(a[:n_avail])[::-1]
    hi, lo = srt[P - 1], srt[P]
    if rel_gap(hi, lo) >= band:
        return set()
    return {c for c in range(n_avail) if a[c] >= lo * (1 - band) and a[c] <= hi * (1 + band)}


def check_retained_valid(row, a, n_avail, P, W, band=NEAR_TIE):
    """A retained set (Eq. 8) that a near-tie at the TopP boundary makes one of several
    correct ones: it holds Recent_W, at most P other cells, every retained non-recent cell
    is at least the P-th norm and every dropped cell at most the (P+1)-th, within the band."""
    R = set(int(c) for c in row)
    assert len(R) == len(row), "retained cells repeat"
    recent = set(range(max(0, n_avail - W), n_avail))
    assert recent <= R, "Recent_W missing from the retained set"
    assert R <= set(range(n_avail)), "retained cell not yet available"
    srt = np.sort(a[:n_avail])[::-1]
    top = R - recent
    assert len(top) <= P
    if n_avail > P and P > 0:
        kth, nxt = srt[P - 1], srt[P]
        for c in top:
            assert a[c] >= kth * (1 - band), f"retained cell {c} below the P-th norm"
        for c in set(range(n_avail)) - R:
            assert a[c] <= nxt * (1 + band) or a[c] <= kth * (1 + band), f"dropped cell {c} above the band"
    assert len(R) >= min(P, n_avail), "fewer than min(P, |C|) cells retained"


def near_tie_reference(sel_row, ref, row, i, p, what):
    """Validate the GPU's selection for one near-tie query (see the module docstring)
    and return the oracle's readout of it, the reference for that query's output."""
    q, k, v, g = ref["inputs"]
    op = ref["prm"]
    blk = i // p.B
    n_avail = oracle.available_count(p.B * blk, p.s)
    A = [int(c) for c in ref["retained"][blk][: ref["n_ret"][blk]]]
    pool = boundary_pool(ref["a"], n_avail, p.P) if p.prune else set()
    if p.prune:
        sure = sorted({c for c in A if c not in pool} | set(range(max(0, n_avail - p.W), n_avail)))
    else:
        sure = A
    reach = set(A) | pool
    S = [int(c) for c in sel_row if c >= 0]
    assert all(c < 0 for c in sel_row[len(S):]), f"{what} query {i}: -1 padding not at the end: {sel_row}"
    assert len(set(S)) == len(S), f"{what} query {i}: repeated cell {sel_row}"
    assert set(S) <= reach, f"{what} query {i}: selected a cell outside its retained set: {sel_row}"
    need = min(p.K, len(sure)) if pool else min(p.K, len(A))
    assert need <= len(S) <= p.K, f"{what} query {i}: {len(S)} cells selected, expected {need}"
    r = {c: oracle.cell_score(q[i], ref["kbar"][c], ref["a"][c], i, c, op) for c in reach}
    m = {c: oracle.cell_score_mag(q[i], ref["kbar"][c], ref["a"][c], i, c, op) for c in reach}

    def at_least(c1, c2):  # r_c1 >= r_c2, or the two within the near-tie band of their term sizes
        return r[c1] >= r[c2] or abs(r[c1] - r[c2]) < NEAR_TIE * max(m[c1], m[c2])

    for t in range(len(S) - 1):
        assert at_least(S[t], S[t + 1]), f"{what} query {i}: selection not in score order {sel_row}"
    for c in S:
        for c2 in sure:
            if c2 not in S:
                assert at_least(c, c2), \
                    f"{what} query {i}: cell {c2} (score {r[c2]!r}) outranks selected {c} ({r[c]!r})"
    return oracle.readout(q[i], k, v, S, g, op)


def lr_reference(sel_gpu, ref, p, i_lo=0, what=""):
    """The oracle's long-range output rows, with every near-tie query's row replaced by the
    oracle's readout of the GPU's (validated) selection.  Returns (rows, n_near_tie)."""
    n = ref["sel"].shape[0]
    tie = excluded_queries(ref, p, i_lo, n)
    out = ref["out"].copy()
    for row in np.nonzero(tie)[0]:
        out[row] = near_tie_reference(sel_gpu[row], ref, row, i_lo + row, p, what)
    return out, int(tie.sum())


def check_output(o, r, dtype, what):
    o = o.astype(np.float64)
    zero_rows = np.all(r == 0, axis=1)
    assert np.all(o[zero_rows] == 0), f"{what}: rows without selection must be exactly zero"
    if dtype == "f32":
        tol = TOL_F32 * np.maximum(1.0, np.abs(r).max(axis=1))
        err = np.abs(o - r).max(axis=1)
        worst = int(np.argmax(err / tol)) if len(err) else 0
        assert np.all(err <= tol), f"{what}: fp32 output error {err[worst]:.3g} > {tol[worst]:.3g}"
    else:
        err = np.abs(o - r)
        assert err.max(initial=0.0) <= TOL_BF16, f"{what}: bf16 output error {err.max():.3g}"


def compare_head(sel_gpu, out_gpu, ref, p, dtype, i_lo=0, what=""):
    """Compare one head's selections and outputs with the oracle: exact where the oracle's
    choice is unique, validated (see the module docstring) at near-ties.  Returns
    (n_exact, n_near_tie); every query is checked."""
    n = ref["sel"].shape[0]
    tie = excluded_queries(ref, p, i_lo, n)
    keep = ~tie
    if sel_gpu is not None:
        bad = np.nonzero(np.any(sel_gpu[keep] != ref["sel"][keep], axis=1))[0]
        if len(bad):
            i = np.nonzero(keep)[0][bad[0]]
            raise AssertionError(f"{what}: selection differs at query {i_lo + i}: gpu {sel_gpu[i]} vs oracle "
                                 f"{ref['sel'][i]} (gap_k {ref['gap_k'][i]:.3g}); {len(bad)} queries differ")
    if out_gpu is not None:
        check_output(out_gpu[keep], ref["out"][keep], dtype, what)
    if tie.any():
        assert sel_gpu is not None and out_gpu is not None and "inputs" in ref, \
            f"{what}: near-tie queries need the GPU's selections, outputs and the oracle inputs"
        for row in np.nonzero(tie)[0]:
            r = near_tie_reference(sel_gpu[row], ref, row, i_lo + row, p, what)
            check_output(out_gpu[row][None], r[None], dtype, f"{what} query {i_lo + row} (near-tie)")
    return int(keep.sum()), int(tie.sum())


def attach(ref, inputs, op):
    """Give an oracle.head result its fp64 inputs (q, k, v, g) and parameters, for
    compare_head's near-tie validation."""
    ref["inputs"] = tuple(inputs)
    ref["prm"] = op
    return ref


# bf16 outputs of this branch are not RMS-normalised and, with alpha_h o_lr added,
# can exceed 8, where one bf16 half-ulp alone is 2^-5: the bound is 2e-2 absolute
# or 0.5% of the reference (about one bf16 ulp), whichever is larger.
TOL_BF16_REL = 5e-3


def check_rows(got, ref, dtype, what, lr_scale=0.0):
    """lr_scale: alpha_h when the long-range output that was added came from the GPU
    (within its own tolerance): Eq. 2 is linear, so its error adds, scaled by alpha_h."""
    got = got.astype(np.float64)
    if dtype == "f32":
        tol = (1.0 + lr_scale) * TOL_F32 * np.maximum(1.0, np.abs(ref).max(axis=1))
        err = np.abs(got - ref).max(axis=1)
        worst = int(np.argmax(err / tol))
        assert np.all(err <= tol), f"{what}: fp32 error {err[worst]:.3g} > {tol[worst]:.3g} at row {worst}"
    else:
        tol = np.maximum(TOL_BF16, TOL_BF16_REL * np.abs(ref)) + lr_scale * TOL_BF16
        err = np.abs(got - ref)
        worst = np.unravel_index(int(np.argmax(err / tol)), err.shape)
        assert np.all(err <= tol), f"{what}: bf16 error {err[worst]:.3g} > {tol[worst]:.3g} at {worst}"
