"""GPU parity of the local RoPE window branch and the branch combination
(fs_local_window) against the fp64 oracle.

FreeSolo, Sec. 3.2 (Eqs. 3-4): causal softmax attention over the last w + 1
tokens with RoPE-rotated queries and keys; Sec. 3.1 (Eq. 2): out = o_sr +
alpha_h o_lr.  Outputs follow the rules of tests/parity_utils.py (fp32: 1e-5
relative per row; bf16: 2e-2 absolute).
"""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import oracle
import synth
from tests import parity_utils as pu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fsl.lib()


def run_case(w, win, base=10000.0, combine=False, in_place=False, heads=None, rows=None, seed=5):
    host = pu.inputs(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    alpha = olr_h = d_olr = None
    if combine:
        r = np.random.default_rng(seed)
        alpha = r.uniform(0.25, 2.0, size=w.H).astype(np.float32)
        olr_h = r.normal(size=(w.batch, w.H, w.N, w.d)).astype(np.float32)
        d_olr = pu.to_device(olr_h, w.dtype) if w.dtype == "f32" else \
            torch.from_numpy(olr_h).cuda().to(torch.bfloat16)
    print(f"[gpu] local {w} w={win} base={base} combine={combine} in_place={in_place}", flush=True)
    out = d_olr if in_place else torch.empty_like(dq)
    fsl.fs_local_window(dq, dk, dv, out, w=win, rope_base=base, alpha=alpha, o_lr=d_olr)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    olr_ref = None if d_olr is None else (d_olr.float().cpu().numpy() if not in_place else None)
    if in_place and combine:
        olr_ref = torch.from_numpy(olr_h).to(torch.bfloat16 if w.dtype == "bf16" else torch.float32).float().numpy()
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    for b, h in heads:
        lo, hi = rows if rows else (0, w.N)
        ref = oracle.local(synth.to_f64(host["q"][b, h], w.dtype), synth.to_f64(host["k"][b, h], w.dtype),
                           synth.to_f64(host["v"][b, h], w.dtype), w=win, rope_base=base,
                           alpha=0.0 if alpha is None else float(alpha[h]),
                           o_lr=None if olr_ref is None else olr_ref[b, h, lo:hi], i_lo=lo, i_hi=hi)
        pu.check_rows(got[b, h, lo:hi], ref, w.dtype, f"local b{b} h{h}")


@pytest.mark.parametrize("w,win", [
    (synth.Workload(batch=2, H=2, N=1000, d=128, dtype="bf16", seed=101, needle_frac=0.005), 512),
    (synth.Workload(batch=1, H=3, N=777, d=64, dtype="bf16", seed=102), 100),
    (synth.Workload(batch=1, H=2, N=600, d=64, dtype="f32", seed=103), 512),
    (synth.Workload(batch=1, H=2, N=700, d=128, dtype="f32", seed=104, needle_frac=0.01), 64),
    (synth.Workload(batch=1, H=2, N=300, d=128, dtype="bf16", seed=105), 0),      # w = 0: o_i = v_i
    (synth.Workload(batch=1, H=2, N=130, d=128, dtype="bf16", seed=106), 5000),   # w >= N: causal, dense
    (synth.Workload(batch=1, H=1, N=1, d=64, dtype="f32", seed=107), 512),        # one token
    (synth.Workload(batch=1, H=2, N=129, d=64, dtype="bf16", seed=108), 31),      # ragged tail, window < tile
], ids=["bf16d128-w512", "bf16d64-w100", "f32d64-w512", "f32d128-w64", "w0", "w-past-N", "N1", "N129-w31"])
def test_local_window(w, win):
    run_case(w, win)


def test_local_rope_base_and_long_positions():
    """Another base, and positions far from 0 (the angles are taken relative to the block start)."""
    run_case(synth.Workload(batch=1, H=2, N=5000, d=128, dtype="bf16", seed=109), 512, base=500000.0,
             rows=(4000, 5000))


@pytest.mark.parametrize("dtype,in_place", [("bf16", False), ("f32", False), ("bf16", True)])
def test_branch_combination_eq2(dtype, in_place):
    """out = o_sr + alpha_h o_lr with per-head alpha (Eq. 2); also written over o_lr in place."""
    w = synth.Workload(batch=2, H=3, N=600, d=128 if dtype == "bf16" else 64, dtype=dtype, seed=110)
    run_case(w, 512, combine=True, in_place=in_place)


def test_local_headline_shape_sampled():
    """b4 H16 d128 N16384 bf16 at w = 512 (the headline prefill's shape): every
    head is computed, sampled heads are checked on the first and last rows."""
    w = synth.WORKLOADS["prefill_16k"]
    run_case(w, 512, heads=[(0, 0), (3, 15)], rows=(16384 - 700, 16384))
    run_case(w, 512, heads=[(1, 7)], rows=(0, 400))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_local_largest_window_sampled(dtype, d):
    """w = 65535, the largest window accepted: each block walks about 2,050 key tiles,
    so the tiles' stepped rotation angles must not drift (they are taken afresh from
    fp64 every 16 tiles).  N = 70,000; the last 96 rows, whose windows are full, and
    rows near the first block boundaries against the oracle."""
    w = synth.Workload(batch=1, H=1, N=70000, d=d, dtype=dtype, seed=113, needle_frac=0.005)
    run_case(w, 65535, rows=(w.N - 96, w.N))
    run_case(w, 65535, rows=(65000, 65200))


def test_local_rejects_window_past_limit():
    q = torch.zeros(1, 1, 64, 64, device="cuda")
    with pytest.raises(fsl.FslError):
        fsl.fs_local_window(q, q, q, q.clone(), w=65536)


def test_local_maximum_length_sampled():
    """N = 2^22, the longest sequence the ABI accepts: the last 300 rows against the oracle."""
    w = synth.Workload(batch=1, H=1, N=1 << 22, d=64, dtype="bf16", seed=112)
    run_case(w, 512, rows=(w.N - 300, w.N))


def test_local_rejects_bad_arguments():
    q = torch.zeros(1, 1, 64, 64, device="cuda")
    with pytest.raises(fsl.FslError):
        fsl.fs_local_window(q, q, q, q.clone(), w=-1)
    with pytest.raises(fsl.FslError):
        fsl.fs_local_window(q, q, q, q.clone(), rope_base=1.0)
    with pytest.raises(fsl.FslError):  # o_lr without alpha
        fsl.fs_local_window(q, q, q, q.clone(), o_lr=q)


@pytest.mark.parametrize("w", [synth.WORKLOADS["prefill_4k"],
                               synth.Workload(batch=1, H=2, N=2500, d=128, dtype="bf16", seed=111,
                                              needle_frac=0.005)],
                         ids=["cfg4k-f32", "bf16d128"])
def test_full_attention_output_end_to_end(w):
    """The whole FreeSolo attention output of Eq. 2: the long-range prefill's output
    (Eqs. 5-9, 17) fed into the local branch with per-head alpha, against the oracle's
    long-range output combined by the oracle's local branch.  At near-tie queries the
    long-range reference is the oracle's readout of the GPU's validated selection."""
    p = fsl.Params()
    host = pu.inputs(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    alpha = np.linspace(0.5, 1.5, w.H).astype(np.float32)
    print(f"[gpu] full attention output {w}", flush=True)
    o_lr, sel, _ = fsl.prefill(dq, dk, dv, p)
    fsl.fs_local_window(dq, dk, dv, o_lr, w=512, alpha=alpha, o_lr=o_lr)  # in place: o_lr becomes o
    torch.cuda.synchronize()
    got = o_lr.float().cpu().numpy()
    sel = sel.cpu().numpy()
    heads = [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads)
    for (b, h), ref in refs.items():
        lr_ref, _ = pu.lr_reference(sel[b, h], ref, p, 0, f"b{b} h{h}")
        full = oracle.local(*(synth.to_f64(host[x][b, h], w.dtype) for x in "qkv"), w=512, alpha=float(alpha[h]),
                            o_lr=lr_ref)
        pu.check_rows(got[b, h], full, w.dtype, f"full output b{b} h{h}", lr_scale=float(alpha[h]))
