"""Shared helpers of the GPU parity tests: seeded inputs on both sides, the oracle
on (sequence, head) samples, and the comparison rules.

Comparison rules (written once, used by every parity test):
  * cell ids (retained sets, selections) are compared exactly, except where the
    oracle reports a near-tie: a relative gap below 1e-6 between the K-th and
    (K+1)-th routing scores of a query, or between the P-th and (P+1)-th key
    norms of a block's prefix.  Such queries are counted and reported.
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


def inputs(w: synth.Workload):
    return {x: synth.tensor(w, x) for x in "qkv"}


def oracle_params(p) -> oracle.Params:
    return oracle.Params(s=p.s, B=p.B, P=p.P, W=p.W, K=p.K, prune=p.prune, eps=p.eps)


def run_oracle(w, host, p, heads, sigma=4.0, lam=1.0, gain=None, i_lo=0, i_hi=None):
    """Oracle results per sampled (b, h) pair (inputs widened exactly to fp64)."""
    op = oracle.Params(s=p.s, B=p.B, P=p.P, W=p.W, K=p.K, prune=p.prune, sigma=sigma, lam=lam, eps=p.eps)

    def one(bh):
        b, h = bh
        g = None if gain is None else gain[h]
        return bh, oracle.head(synth.to_f64(host["q"][b, h], w.dtype), synth.to_f64(host["k"][b, h], w.dtype),
                               synth.to_f64(host["v"][b, h], w.dtype), g, op, i_lo, i_hi)

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return dict(ex.map(one, heads))


def excluded_queries(ref, p, i_lo, n):
    """Queries whose selection is decided by a near-tie (see module docstring)."""
    gap_k = ref["gap_k"]
    blocks = (np.arange(i_lo, i_lo + n) // p.B)
    gap_p = ref["gap_p"][blocks]
    return (gap_k < NEAR_TIE) | (np.nan_to_num(gap_p, nan=np.inf) < NEAR_TIE)


def compare_head(sel_gpu, out_gpu, ref, p, dtype, i_lo=0, what=""):
    """Compare one head's selections and outputs; returns (n_checked, n_near_tie)."""
    n = ref["sel"].shape[0]
    skip = excluded_queries(ref, p, i_lo, n)
    keep = ~skip
    if sel_gpu is not None:
        bad = np.nonzero(np.any(sel_gpu[keep] != ref["sel"][keep], axis=1))[0]
        if len(bad):
            i = np.nonzero(keep)[0][bad[0]]
            raise AssertionError(f"{what}: selection differs at query {i_lo + i}: gpu {sel_gpu[i]} vs oracle "
                                 f"{ref['sel'][i]} (gap_k {ref['gap_k'][i]:.3g}); {len(bad)} queries differ")
    if out_gpu is not None:
        o = out_gpu[keep].astype(np.float64)
        r = ref["out"][keep]
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
    return int(keep.sum()), int(skip.sum())


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
