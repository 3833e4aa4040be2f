"""GPU parity of FS-B (fs_fsb_prefill: FreeSolo Sec. 3.4; App. E.1) against the
fp64 oracle (oracle/fsb_oracle.c) on the same seeded inputs.

Rules:
  * candidates B_i and selections are compared exactly, except at a near-tie:
    a beam cut (the last child kept vs the first dropped, any level, either
    forest) or the K/K+1 rerank boundary within 1e-6 of the larger term size,
    or a median split of the block's forests within 1e-9 (the trees are built
    in fp64 on both sides).  A near-tie query is validated instead: its cells
    must be distinct cells available to the query, and its output must match
    the oracle's readout of the GPU's own selection.  Near-ties are counted and
    capped at 1% of the queries.
  * outputs: as for the long-range branch (fp32: 1e-5 relative per row; bf16:
    2e-2 absolute), rows without a selection exactly zero.
tau_h is the median cell norm of a separate calibration window per head (the
page calibrates it once per checkpoint as a median cell norm).
"""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import oracle
import synth
from tests import parity_utils as pu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPLIT_TIE = 1e-9


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fsl.lib()


def calibrated_tau(w, s=32):
    """Per head: the median cell norm of a 4096-token window drawn like the workload's keys
    with another seed (the page's calibration uses separate text)."""
    cal = synth.Workload(batch=1, H=w.H, N=4096, d=w.d, dtype=w.dtype, seed=w.seed + 1000,
                         needle_frac=w.needle_frac)
    kc = synth.tensor(cal, "k")
    taus = []
    for h in range(w.H):
        _, a = oracle.cell_summaries(synth.to_f64(kc[0, h], w.dtype), oracle.Params(s=s))
        taus.append(float(np.float32(np.median(a))))
    return taus


def near_ties(ref):
    return (ref["gap_beam"] < pu.NEAR_TIE) | (ref["gap_rerank"] < pu.NEAR_TIE) | (ref["gap_split"] < SPLIT_TIE)


def check_fsb(w, p=fsl.Params(), fb=fsl.FsbParams(), heads=None, lam=1.0, sigma=4.0, gain=None, tau=None,
              i_lo=0, i_hi=None, max_tie_frac=0.01):
    host = pu.inputs(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    taus = tau if tau is not None else calibrated_tau(w)
    g = None if gain is None else torch.from_numpy(gain).cuda()
    print(f"[gpu] fsb {w} {p} {fb} tau={taus[:2]}", flush=True)
    out, sel, cand, _ = fsl.fsb_prefill(dq, dk, dv, taus, p, fb, sigma=sigma, lam=lam, gain=g, want_cand=True)
    torch.cuda.synchronize()
    out, sel, cand = out.float().cpu().numpy(), sel.cpu().numpy(), cand.cpu().numpy()
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    i_hi = w.N if i_hi is None else i_hi
    exact = ties = 0
    for b, h in heads:
        x = tuple(synth.to_f64(host[t][b, h], w.dtype) for t in "qkv")
        op = pu.oracle_params(p, sigma, lam)
        ofb = oracle.FsbParams(tau=float(taus[h]), Wb=fb.Wb, c=fb.c)
        gh = None if gain is None else gain[h]
        ref = oracle.fsb_head(*x, gh, op, ofb, i_lo, i_hi)
        tie = near_ties(ref)
        keep = ~tie
        what = f"FS-B {w} b{b} h{h}"
        rows = np.arange(i_lo, i_hi)
        bad = np.nonzero(np.any(cand[b, h, rows][keep] != ref["cand"][keep], axis=1))[0]
        if len(bad):
            r = np.nonzero(keep)[0][bad[0]]
            raise AssertionError(f"{what}: candidates differ at query {i_lo + r}: gpu {cand[b, h, i_lo + r]} vs "
                                 f"oracle {ref['cand'][r]}; {len(bad)} queries differ")
        bad = np.nonzero(np.any(sel[b, h, rows][keep] != ref["sel"][keep], axis=1))[0]
        if len(bad):
            r = np.nonzero(keep)[0][bad[0]]
            raise AssertionError(f"{what}: selection differs at query {i_lo + r}: gpu {sel[b, h, i_lo + r]} vs "
                                 f"oracle {ref['sel'][r]} (rerank gap {ref['gap_rerank'][r]:.3g}); {len(bad)} differ")
        pu.check_output(out[b, h, rows][keep], ref["out"][keep], w.dtype, what)
        for r in np.nonzero(tie)[0]:
            i = i_lo + r
            S = [int(c) for c in sel[b, h, i] if c >= 0]
            n_avail = (i // p.B) * (p.B // p.s)
            assert len(set(S)) == len(S) and all(0 <= c < n_avail for c in S), f"{what} query {i}: {sel[b, h, i]}"
            ro = oracle.readout(x[0][i], x[1], x[2], S, gh, op)
            pu.check_output(out[b, h, i][None], ro[None], w.dtype, f"{what} query {i} (near-tie)")
        exact += int(keep.sum())
        ties += int(tie.sum())
    print(f"checked {exact} queries exactly, {ties} near-ties validated")
    assert ties <= max_tie_frac * (exact + ties)
    return out, sel, cand


@pytest.mark.parametrize("w,p,fb,extra", [
    (synth.Workload(batch=1, H=2, N=1024, d=64, dtype="f32", seed=401), fsl.Params(), fsl.FsbParams(), {}),
    (synth.Workload(batch=1, H=2, N=2048, d=128, dtype="bf16", seed=402, needle_frac=0.01), fsl.Params(),
     fsl.FsbParams(Wb=4), {}),
    (synth.Workload(batch=2, H=2, N=3000, d=64, dtype="bf16", seed=403, needle_frac=0.005), fsl.Params(),
     fsl.FsbParams(), {}),
    (synth.Workload(batch=1, H=2, N=4096, d=128, dtype="bf16", seed=404, needle_frac=0.005), fsl.Params(),
     fsl.FsbParams(), {}),
    (synth.Workload(batch=1, H=2, N=2500, d=128, dtype="f32", seed=405, needle_frac=0.01), fsl.Params(K=8),
     fsl.FsbParams(Wb=6, c=2.0), {"gain": True}),
    (synth.Workload(batch=1, H=2, N=2048, d=64, dtype="bf16", seed=406), fsl.Params(), fsl.FsbParams(Wb=1), {}),
    (synth.Workload(batch=1, H=2, N=2048, d=128, dtype="bf16", seed=407, needle_frac=0.01), fsl.Params(),
     fsl.FsbParams(c=0.0), {}),
    (synth.Workload(batch=1, H=2, N=2048, d=64, dtype="f32", seed=408, needle_frac=0.01), fsl.Params(K=3),
     fsl.FsbParams(Wb=8), {"lam": 0.0}),
    (synth.Workload(batch=1, H=2, N=1500, d=128, dtype="bf16", seed=409), fsl.Params(), fsl.FsbParams(Wb=5),
     {"tau": [1e30, 1e30]}),  # second forest empty
    (synth.Workload(batch=1, H=2, N=1500, d=64, dtype="bf16", seed=410), fsl.Params(), fsl.FsbParams(Wb=5),
     {"tau": [0.0, 0.0]}),    # second forest = first
    (synth.Workload(batch=1, H=3, N=1300, d=128, dtype="f32", seed=411, needle_frac=0.01), fsl.Params(K=1),
     fsl.FsbParams(Wb=3), {"sigma": 40.0, "lam": 0.3}),
], ids=["f32d64-1k", "bf16d128-Wb4", "bf16d64-ragged", "bf16d128-4k", "f32d128-K8-gain", "Wb1", "c0", "lam0-K3",
        "tau-empty", "tau-all", "K1-sigma40"])
def test_fsb_prefill(w, p, fb, extra):
    gain = synth.gains(96, w.H, w.d) if extra.get("gain") else None
    check_fsb(w, p, fb, lam=extra.get("lam", 1.0), sigma=extra.get("sigma", 4.0), gain=gain, tau=extra.get("tau"))


@pytest.mark.parametrize("N", [1, 127, 128, 129, 160, 700])
def test_fsb_tiny_and_ragged(N):
    w = synth.Workload(batch=1, H=2, N=N, d=64, dtype="bf16", seed=420 + N, needle_frac=0.02)
    out, sel, cand = check_fsb(w, fsl.Params(), fsl.FsbParams(Wb=3))
    assert np.all(sel[:, :, :min(N, 128)] == -1) and np.all(out[:, :, :min(N, 128)] == 0)


def test_fsb_headline_shape_sampled():
    """b4 H16 d128 N16384 bf16 (the headline prefill's shape), the page's W^b = 16 and
    c = 8: the whole batch on the GPU, every query of two sampled heads against the oracle."""
    w = synth.WORKLOADS["prefill_16k"]
    check_fsb(w, fsl.Params(), fsl.FsbParams(), heads=[(0, 3), (3, 12)])


def test_fsb_largest_forest_sampled():
    """N = 131,200, the longest sequence FS-B accepts (4096 cells available to the last
    block, a forest of one 4096-cell chunk): the queries of an early, a middle and the last
    block against the oracle."""
    w = synth.Workload(batch=1, H=1, N=131200, d=64, dtype="bf16", seed=430, needle_frac=0.005)
    host = pu.inputs(w)
    taus = calibrated_tau(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    print(f"[gpu] fsb largest forest {w}", flush=True)
    out, sel, cand, _ = fsl.fsb_prefill(dq, dk, dv, taus, fsl.Params(), fsl.FsbParams(), want_cand=True)
    torch.cuda.synchronize()
    out, sel, cand = out.float().cpu().numpy(), sel.cpu().numpy(), cand.cpu().numpy()
    x = tuple(synth.to_f64(host[t][0, 0], w.dtype) for t in "qkv")
    del host
    ties = total = 0
    for lo in (128 * 40, 128 * 512, w.N - 128):
        ref = oracle.fsb_head(*x, None, pu.oracle_params(fsl.Params()), oracle.FsbParams(tau=taus[0]), lo, lo + 128)
        tie = near_ties(ref)
        keep = ~tie
        np.testing.assert_array_equal(cand[0, 0, lo:lo + 128][keep], ref["cand"][keep])
        np.testing.assert_array_equal(sel[0, 0, lo:lo + 128][keep], ref["sel"][keep])
        pu.check_output(out[0, 0, lo:lo + 128][keep], ref["out"][keep], w.dtype, f"block {lo // 128}")
        ties += int(tie.sum())
        total += 128
    assert ties <= 0.01 * total


def test_fsb_deterministic():
    w = synth.Workload(batch=1, H=2, N=2048, d=128, dtype="bf16", seed=440, needle_frac=0.005)
    host = pu.inputs(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    taus = calibrated_tau(w)
    o1, s1, c1, ws = fsl.fsb_prefill(dq, dk, dv, taus, want_cand=True)
    o2, s2, c2, _ = fsl.fsb_prefill(dq, dk, dv, taus, want_cand=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(c1, c2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))
