"""GPU parity of the local branch's streaming decode (fs_local_state_build,
fs_local_decode) against the fp64 oracle.

FreeSolo, Sec. 3.2 (Eqs. 3-4): the query at position i attends to the tokens
[max(0, i - w), i] with RoPE (relative form); Sec. 3.1 (Eq. 2): out = o_sr +
alpha_h o_lr.  A decode step's output must equal row i of the local branch over
the whole sequence, which is what the oracle computes; outputs follow the rules
of tests/parity_utils.py (check_rows).
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


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def steps_of(a, dtype):
    """[b, H, T, d] host rows -> [T, b, H, d] on the device, contiguous per step."""
    return pu.to_device(np.ascontiguousarray(np.moveaxis(a, 2, 0)), dtype)


def run_steps(w, host, win, N0, T, base=10000.0, n_given=None, combine=True, seed=7, in_place=False):
    """State from the n_given tokens before N0 (default: all N0), then T steps.
    host arrays cover positions [lo, lo + rows) with lo = N0 - n_given.
    Returns (out [b, H, T, d] fp64, o_lr [b, H, T, d] as passed, alpha or None)."""
    n = N0 if n_given is None else n_given
    lo = N0 - n
    dt = torch_dtype(w.dtype)
    state = fsl.new_local_state(w.batch, w.H, w.d, dt, w=win)
    state.zero_()  # padding bytes too, so that whole states compare equal
    dk, dv = (pu.to_device(np.ascontiguousarray(host[x][:, :, :n]), w.dtype) for x in "kv")
    print(f"[gpu] local decode {w} w={win} N0={N0} n={n} T={T} base={base} combine={combine}", flush=True)
    fsl.fs_local_state_build(state, dk, dv, pos=N0, w=win, rope_base=base)
    st = {x: steps_of(host[x][:, :, n:n + T], w.dtype) for x in "qkv"}
    alpha = olr = d_olr = None
    if combine:
        r = np.random.default_rng(seed)
        alpha = r.uniform(0.25, 2.0, size=w.H).astype(np.float32)
        olr = r.normal(size=(T, w.batch, w.H, w.d)).astype(np.float32)
        d_olr = torch.from_numpy(olr).cuda().to(dt)
        olr = d_olr.float().cpu().numpy()  # what the kernel reads
    outs = d_olr if in_place else torch.empty(T, w.batch, w.H, w.d, dtype=dt, device="cuda")
    for t in range(T):
        fsl.fs_local_decode(state, st["q"][t], st["k"][t], st["v"][t], outs[t], w=win, alpha=alpha,
                            o_lr=None if d_olr is None else d_olr[t])
    torch.cuda.synchronize()
    got = np.moveaxis(outs.float().cpu().numpy(), 0, 2)
    return got, (None if olr is None else np.moveaxis(olr, 0, 2)), alpha, state, lo


def check_steps(w, host, win, N0, T, got, olr, alpha, lo=0, base=10000.0, heads=None):
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    for b, h in heads:
        ref = oracle.local(*(synth.to_f64(host[x][b, h], w.dtype) for x in "qkv"), w=win, rope_base=base,
                           alpha=0.0 if alpha is None else float(alpha[h]),
                           o_lr=None if olr is None else olr[b, h], i_lo=N0 - lo, i_hi=N0 - lo + T)
        pu.check_rows(got[b, h], ref, w.dtype, f"local decode b{b} h{h}")


@pytest.mark.parametrize("w,win,N0,T", [
    (synth.Workload(batch=2, H=2, N=760, d=128, dtype="bf16", seed=201, needle_frac=0.005), 512, 700, 60),
    (synth.Workload(batch=1, H=3, N=230, d=64, dtype="bf16", seed=202), 100, 50, 180),   # fills, then wraps
    (synth.Workload(batch=1, H=2, N=200, d=64, dtype="f32", seed=203), 64, 100, 100),
    (synth.Workload(batch=1, H=2, N=150, d=128, dtype="f32", seed=204), 512, 20, 130),   # window never full
    (synth.Workload(batch=1, H=2, N=40, d=128, dtype="bf16", seed=205), 7, 0, 40),       # empty prefix, many wraps
    (synth.Workload(batch=1, H=2, N=30, d=64, dtype="f32", seed=206), 0, 10, 20),        # w = 0: o_i = v_i
    (synth.Workload(batch=1, H=2, N=1600, d=128, dtype="bf16", seed=211), 1100, 1500, 100),  # three passes
    (synth.Workload(batch=1, H=2, N=900, d=128, dtype="f32", seed=212), 300, 820, 80),   # two passes, full
    (synth.Workload(batch=1, H=2, N=700, d=64, dtype="bf16", seed=213), 515, 300, 300),  # fills past one pass
], ids=["bf16d128-w512", "bf16d64-w100-wrap", "f32d64-w64", "f32d128-short", "empty-prefix-w7", "w0",
        "bf16d128-w1100", "f32d128-w300", "bf16d64-w515-fill"])
def test_local_decode_stream(w, win, N0, T):
    host = pu.inputs(w)
    got, olr, alpha, _, _ = run_steps(w, host, win, N0, T)
    check_steps(w, host, win, N0, T, got, olr, alpha)


def test_local_decode_without_combination():
    w = synth.Workload(batch=1, H=2, N=600, d=128, dtype="bf16", seed=207)
    host = pu.inputs(w)
    got, olr, alpha, _, _ = run_steps(w, host, 512, 560, 40, combine=False)
    check_steps(w, host, 512, 560, 40, got, olr, alpha)


def test_local_decode_in_place_over_o_lr():
    w = synth.Workload(batch=2, H=2, N=300, d=64, dtype="bf16", seed=208)
    host = pu.inputs(w)
    got, olr, alpha, _, _ = run_steps(w, host, 128, 250, 50, in_place=True)
    check_steps(w, host, 128, 250, 50, got, olr, alpha)


def test_local_decode_from_prompt_tail_and_base():
    """A state built from only the last w tokens of a long prompt, positions far from
    0 and another RoPE base: the same rows as the whole sequence."""
    w = synth.Workload(batch=1, H=2, N=5040, d=128, dtype="f32", seed=209)
    host = pu.inputs(w)
    N0, T, win = 5000, 40, 512
    tail = {x: np.ascontiguousarray(host[x][:, :, N0 - win:]) for x in "qkv"}
    got, olr, alpha, _, lo = run_steps(w, tail, win, N0, T, base=500000.0, n_given=win)
    check_steps(w, host, win, N0, T, got, olr, alpha, lo=0, base=500000.0)


def test_local_decode_headline_shape_sampled():
    """b32 H8 d128 bf16 after a 262,144-token prefix (the streaming-decode shape):
    the state is built from the prefix's last 512 tokens; sampled heads are checked
    against the oracle on the window's rows, which RoPE's relative form (Eq. 3)
    makes independent of where they sit."""
    w = synth.WORKLOADS["decode_256k"]
    N0, T, win = 262144, 3, 512
    lo = N0 - win
    host = {x: synth.tensor(w, x, lo, N0 + T) for x in "qkv"}
    got, olr, alpha, _, _ = run_steps(w, host, win, N0, T, n_given=win)
    check_steps(w, host, win, N0, T, got, olr, alpha, lo=lo, heads=[(0, 0), (13, 5), (31, 7)])


def test_local_decode_graph_replay():
    """Steps captured in a HIP graph, replayed from a restored state, equal eager steps."""
    w = synth.Workload(batch=2, H=2, N=300, d=128, dtype="bf16", seed=210)
    host = pu.inputs(w)
    N0, T, win = 200, 16, 64
    got, olr, alpha, state, _ = run_steps(w, host, win, N0, T)
    snap = fsl.new_local_state(w.batch, w.H, w.d, torch.bfloat16, w=win)
    snap.zero_()
    fsl.fs_local_state_build(snap, pu.to_device(np.ascontiguousarray(host["k"][:, :, :N0]), "bf16"),
                             pu.to_device(np.ascontiguousarray(host["v"][:, :, :N0]), "bf16"), pos=N0, w=win)
    st = {x: steps_of(host[x][:, :, N0:N0 + T], "bf16") for x in "qkv"}
    d_olr = torch.from_numpy(np.ascontiguousarray(np.moveaxis(olr, 2, 0))).cuda().to(torch.bfloat16)
    work = torch.empty_like(snap)
    outs = torch.empty(T, w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for t in range(T):
                fsl.fs_local_decode(work, st["q"][t], st["k"][t], st["v"][t], outs[t], w=win, alpha=alpha,
                                    o_lr=d_olr[t], stream=cap.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        work.copy_(snap)
        outs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rep_out = np.moveaxis(outs.float().cpu().numpy(), 0, 2)
        assert np.array_equal(rep_out, got), f"replay {rep} differs from the eager steps"
        assert torch.equal(work, state), f"replay {rep}: state differs from the eager state"


def test_local_decode_rejects_foreign_state():
    """A buffer of the right size that was not built for this shape: NaN out, state untouched."""
    b, H, d, win = 1, 2, 64, 32
    state = fsl.new_local_state(b, H, d, torch.float32, w=win)
    state.zero_()
    q = torch.ones(b, H, d, device="cuda")
    out = torch.zeros_like(q)
    fsl.fs_local_decode(state, q, q, q, out, w=win)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert int(state.count_nonzero()) == 0
    # a state for another w has another size: rejected on the host
    with pytest.raises(fsl.FslError):
        fsl.fs_local_decode(state, q, q, q, out, w=win + 1)


@pytest.mark.parametrize("needles", [0.0, 0.005], ids=["plain", "needles"])
def test_local_decode_largest_window(needles):
    """w = 65535, the largest window the ABI accepts (a 65,536-row table and rings).  With
    needle keys the softmax is peaked, which is where a single running fp32 sum over the
    2,048 rows of a group would lose up to 1e-4 of the output."""
    w = synth.Workload(batch=1, H=1, N=65540, d=64, dtype="f32", seed=214, needle_frac=needles)
    host = pu.inputs(w)
    got, olr, alpha, _, _ = run_steps(w, host, 65535, 65537, 3)
    check_steps(w, host, 65535, 65537, 3, got, olr, alpha)


def test_full_attention_decode_output():
    """The whole FreeSolo attention output at decode (Eq. 2): every step's long-range
    output (fs_longrange_decode: Eqs. 5-9, 15, 17) is fed into the local decode with a
    per-head alpha, against the oracle's long-range rows combined by the oracle's local
    branch.  At steps whose long-range selection is decided by a near-tie the reference
    reads out the GPU's validated selection; the long-range output's own tolerance is
    added, scaled by alpha_h (Eq. 2 is linear)."""
    w = synth.Workload(batch=2, H=2, N=1400, d=128, dtype="bf16", seed=215, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    N0, T, win = 1000, 120, 512
    host = pu.inputs(w)
    dk, dv = (pu.to_device(np.ascontiguousarray(host[x][:, :, :N0]), w.dtype) for x in "kv")
    print(f"[gpu] full attention decode {w} {p} N0={N0} T={T} w={win}", flush=True)
    lr_state = fsl.new_state(w.batch, w.H, w.d, torch.bfloat16, p)
    fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=lr_state)
    loc_state = fsl.new_local_state(w.batch, w.H, w.d, torch.bfloat16, w=win)
    fsl.fs_local_state_build(loc_state, dk, dv, pos=N0, w=win)
    st = {x: steps_of(host[x][:, :, N0:N0 + T], w.dtype) for x in "qkv"}
    alpha = np.linspace(0.5, 1.5, w.H).astype(np.float32)
    outs = torch.empty(T, w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    sels = torch.empty(T, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")
    for t in range(T):
        o_lr, _ = fsl.decode(lr_state, st["q"][t], st["k"][t], st["v"][t], p, sel=sels[t])
        fsl.fs_local_decode(loc_state, st["q"][t], st["k"][t], st["v"][t], outs[t], w=win, alpha=alpha, o_lr=o_lr)
    torch.cuda.synchronize()
    got = np.moveaxis(outs.float().cpu().numpy(), 0, 2)
    sel = np.moveaxis(sels.cpu().numpy(), 0, 2)
    heads = [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, i_lo=N0, i_hi=N0 + T)
    ties = 0
    for (b, h), ref in refs.items():
        lr_ref, n_tie = pu.lr_reference(sel[b, h], ref, p, N0, f"decode b{b} h{h}")
        ties += n_tie
        full = oracle.local(*(synth.to_f64(host[x][b, h], w.dtype) for x in "qkv"), w=win, alpha=float(alpha[h]),
                            o_lr=lr_ref, i_lo=N0, i_hi=N0 + T)
        pu.check_rows(got[b, h], full, w.dtype, f"full decode output b{b} h{h}", lr_scale=float(alpha[h]))
    assert ties <= 0.01 * len(heads) * T


def test_local_decode_largest_grid():
    """batch * H = 65,408 (b511 H128) records, w = 64: one step, sampled records
    against the oracle."""
    w = synth.Workload(batch=511, H=128, N=161, d=64, dtype="bf16", seed=216)
    host = pu.inputs(w)
    got, olr, alpha, _, _ = run_steps(w, host, 64, 160, 1)
    check_steps(w, host, 64, 160, 1, got, olr, alpha, heads=[(0, 0), (255, 64), (510, 127)])
