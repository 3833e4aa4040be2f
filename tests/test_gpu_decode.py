"""GPU parity of streaming decode (fs_longrange_decode) against the fp64 oracle.

The page defines decoding as the same causal operator as prompt prefill (FreeSolo,
Sec. 3.3 "Inference"), so the reference for a decode step at position i is the
oracle's prefill output at i over the whole sequence.  Each case builds a state
with a prefill of N0 tokens, feeds T more tokens one step at a time, and compares
every step's selection (exact; near-ties validated) and output (tolerance) with the
oracle at positions N0 .. N0+T-1; see tests/parity_utils.py for the rules.
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


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def run_stream(w, host, p, N0, T, sigma=4.0, lam=1.0, gain=None, state_only=True):
    """Prefill N0 tokens into a fresh state, then T decode steps; returns (out [b,H,T,d], sel [b,H,T,K], state)."""
    dq, dk, dv = (pu.to_device(np.ascontiguousarray(host[x][:, :, :N0]), w.dtype) for x in "qkv")
    g = None if gain is None else torch.from_numpy(gain).cuda()
    state = fsl.new_state(w.batch, w.H, w.d, torch_dtype(w), p)
    print(f"[gpu] decode stream {w} {p} N0={N0} T={T}", flush=True)
    if state_only:
        fsl.prefill(None, dk, None if dv is None else dv, p, sigma=sigma, lam=lam, gain=g, want_out=False,
                    want_sel=False, state=state)
    else:
        fsl.prefill(dq, dk, dv, p, sigma=sigma, lam=lam, gain=g, state=state)
    # per-step inputs [T, b, H, d], contiguous per step
    steps = {x: pu.to_device(np.ascontiguousarray(np.moveaxis(host[x][:, :, N0:N0 + T], 2, 0)), w.dtype)
             for x in "qkv"}
    outs = torch.empty(T, w.batch, w.H, w.d, dtype=torch_dtype(w), device="cuda")
    sels = torch.empty(T, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")
    for t in range(T):
        fsl.decode(state, steps["q"][t], steps["k"][t], steps["v"][t], p, sigma=sigma, lam=lam, gain=g,
                   out=outs[t], sel=sels[t])
    torch.cuda.synchronize()
    out = np.moveaxis(outs.float().cpu().numpy(), 0, 2)
    sel = np.moveaxis(sels.cpu().numpy(), 0, 2)
    return out, sel, state


def check_stream(w, p, N0, T, heads=None, sigma=4.0, lam=1.0, gain=None, state_only=True, max_skip_frac=0.01):
    assert w.N >= N0 + T
    host = pu.inputs(w)
    out, sel, state = run_stream(w, host, p, N0, T, sigma, lam, gain, state_only)
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, sigma, lam, gain, i_lo=N0, i_hi=N0 + T)
    checked = skipped = 0
    for (b, h), ref in refs.items():
        c, s = pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, i_lo=N0,
                               what=f"decode {w.name or w} b{b} h{h}")
        checked += c
        skipped += s
    print(f"checked {checked} decode steps exactly, {skipped} near-ties validated")
    assert skipped <= max_skip_frac * (checked + skipped)
    return out, sel, state


@pytest.mark.parametrize("w,p,N0,T,extra", [
    # mid-cell, mid-block start; pruning active (|C| > P) for most steps
    (synth.Workload(batch=2, H=2, N=1700, d=128, dtype="bf16", seed=81, needle_frac=0.01), fsl.Params(P=6, W=2),
     1000, 700, {}),
    # block-aligned start: the very first step merges
    (synth.Workload(batch=1, H=3, N=1600, d=64, dtype="f32", seed=82, needle_frac=0.01), fsl.Params(P=5, W=3),
     1024, 520, {}),
    # cell-aligned, not block-aligned; no recent window
    (synth.Workload(batch=1, H=2, N=1500, d=128, dtype="f32", seed=83), fsl.Params(P=8, W=0), 992, 500, {}),
    # start inside the first block (empty retained set at first), K=3
    (synth.Workload(batch=1, H=2, N=600, d=64, dtype="bf16", seed=84, needle_frac=0.02), fsl.Params(P=4, W=1, K=3),
     100, 480, {}),
    # a single prompt token
    (synth.Workload(batch=1, H=2, N=400, d=64, dtype="f32", seed=85), fsl.Params(P=3, W=2), 1, 390, {}),
    # recent window only (P = 0)
    (synth.Workload(batch=1, H=2, N=900, d=64, dtype="f32", seed=86), fsl.Params(P=0, W=4), 300, 560, {}),
    # nothing retained at all (P = W = 0): every output is zero
    (synth.Workload(batch=1, H=2, N=500, d=64, dtype="bf16", seed=87), fsl.Params(P=0, W=0), 200, 300, {}),
    # K = 8 (two gather rounds per wave), gains, prefill with outputs as well
    (synth.Workload(batch=1, H=2, N=1400, d=128, dtype="bf16", seed=88, needle_frac=0.01),
     fsl.Params(P=12, W=4, K=8), 777, 600, {"gain": True, "state_only": False}),
    # content-only routing (lambda = 0) and another sigma
    (synth.Workload(batch=1, H=2, N=1300, d=64, dtype="f32", seed=89, needle_frac=0.01), fsl.Params(P=7, W=2),
     640, 600, {"lam": 0.0}),
    (synth.Workload(batch=1, H=2, N=1300, d=128, dtype="bf16", seed=90), fsl.Params(P=7, W=2), 700, 500,
     {"sigma": 40.0, "lam": 0.3}),
    # the page's budgets P=64, W=8 past the point where pruning binds (> 72 cells)
    (synth.Workload(batch=1, H=2, N=3000, d=128, dtype="bf16", seed=91, needle_frac=0.005), fsl.Params(),
     2300, 700, {}),
    # largest supported slot count: P + W + B/s = 128
    (synth.Workload(batch=1, H=1, N=4800, d=64, dtype="f32", seed=92, needle_frac=0.01), fsl.Params(P=100, W=24),
     4000, 800, {}),
], ids=["bf16d128-mid", "f32d64-aligned", "f32d128-W0", "bf16d64-block0-K3", "N0eq1", "P0W4", "P0W0",
        "K8-gain", "lam0", "sigma40", "P64W8", "S128"])
def test_decode_stream(w, p, N0, T, extra):
    gain = synth.gains(98, w.H, w.d) if extra.get("gain") else None
    out, sel, _ = check_stream(w, p, N0, T, sigma=extra.get("sigma", 4.0), lam=extra.get("lam", 1.0), gain=gain,
                               state_only=extra.get("state_only", True))
    if p.P == 0 and p.W == 0:
        assert np.all(sel == -1) and np.all(out == 0)


def test_decode_equals_prefill_selection():
    """Decoding positions N0.. of a sequence selects the same cells as prefilling the
    whole sequence (both are the same causal operator)."""
    w = synth.Workload(batch=2, H=4, N=4096 + 300, d=128, dtype="bf16", seed=93, needle_frac=0.005)
    p = fsl.Params()
    host = pu.inputs(w)
    N0 = 4096 - 57
    T = w.N - N0
    _, sel_dec, _ = run_stream(w, host, p, N0, T)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    _, sel_pre, _ = fsl.prefill(dq, dk, dv, p)
    sel_pre = sel_pre[:, :, N0:].cpu().numpy()
    refs = pu.run_oracle(w, host, p, [(0, 0), (1, 3)], i_lo=N0, i_hi=w.N)
    for (b, h), ref in refs.items():
        ok = ~pu.excluded_queries(ref, p, N0, T)
        np.testing.assert_array_equal(sel_dec[b, h][ok], sel_pre[b, h][ok])
    diff = np.any(sel_dec != sel_pre, axis=-1).mean()
    assert diff < 1e-3, f"decode and prefill selections differ on {diff:.2%} of steps"


def test_decode_resume_bitwise():
    """Copying the state's bytes checkpoints the stream: a copy continued later gives
    bitwise the same outputs as the original."""
    w = synth.Workload(batch=2, H=2, N=1600, d=128, dtype="bf16", seed=94, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    host = pu.inputs(w)
    N0, T1, T2 = 700, 333, 400
    _, _, state = run_stream(w, host, p, N0, T1)
    snap = state.clone()
    steps = {x: pu.to_device(np.ascontiguousarray(np.moveaxis(host[x][:, :, N0 + T1:N0 + T1 + T2], 2, 0)), w.dtype)
             for x in "qkv"}

    def cont(st):
        outs, sels = [], []
        for t in range(T2):
            o, s = fsl.decode(st, steps["q"][t], steps["k"][t], steps["v"][t], p)
            outs.append(o)
            sels.append(s)
        torch.cuda.synchronize()
        return torch.stack(outs).cpu(), torch.stack(sels).cpu()

    o1, s1 = cont(state)
    o2, s2 = cont(snap)
    assert torch.equal(s1, s2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # and the uninterrupted stream gives the same
    out_full, sel_full, _ = run_stream(w, host, p, N0, T1 + T2)
    np.testing.assert_array_equal(np.moveaxis(s1.numpy(), 0, 2), sel_full[:, :, T1:])
    np.testing.assert_array_equal(np.moveaxis(o1.float().numpy(), 0, 2), out_full[:, :, T1:])


def test_decode_graph_replay():
    """Decode steps captured in a HIP graph replay to the eager results (the state is
    restored from a snapshot before each replay; eager work runs in between)."""
    w = synth.Workload(batch=2, H=4, N=1200, d=128, dtype="bf16", seed=95, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    host = pu.inputs(w)
    N0, T = 1000, 140  # crosses the block boundary at 1024 and 1152 and several cell ends
    _, _, state = run_stream(w, host, p, N0, 0)
    snap = state.clone()
    steps = {x: pu.to_device(np.ascontiguousarray(np.moveaxis(host[x][:, :, N0:N0 + T], 2, 0)), w.dtype)
             for x in "qkv"}
    outs = torch.empty(T, w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    sels = torch.empty(T, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")

    def run_all():
        for t in range(T):
            fsl.decode(state, steps["q"][t], steps["k"][t], steps["v"][t], p, out=outs[t], sel=sels[t])

    run_all()
    torch.cuda.synchronize()
    ref_o, ref_s = outs.clone(), sels.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        state.copy_(snap)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(snap)
        outs.zero_()
        sels.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sels, ref_s), f"replay {rep}: selections differ"
        assert torch.equal(outs.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: outputs differ"


def test_decode_rejects_foreign_state():
    """A buffer of the right size that no prefill filled: outputs are NaN, selections -1,
    and the buffer is left untouched."""
    p = fsl.Params()
    b, H, d = 2, 3, 64
    state = fsl.new_state(b, H, d, torch.float32, p)
    state.zero_()
    q = torch.randn(b, H, d, device="cuda")
    o, s = fsl.decode(state, q, q, q, p)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and (s == -1).all()
    assert int(state.count_nonzero()) == 0


def test_decode_full_length_sampled():
    """The decode workload's shape per sequence (H=8, d=128, a 262,144-token prefix,
    bf16) for two sequences: state from a state-only prefill, 130 steps (a block's
    merge at the first step and one more at step 128), every step of two heads
    against the oracle."""
    w0 = synth.WORKLOADS["decode_256k"]
    w = synth.Workload(batch=2, H=8, N=w0.N + 2, d=w0.d, dtype=w0.dtype, seed=w0.seed,
                       needle_frac=w0.needle_frac)
    N0 = 262144
    check_stream(w, fsl.Params(), N0, 130, heads=[(0, 1), (1, 6)])


def test_decode_per_head_constants():
    """Every head with its own sigma_h and lambda_h (Eq. 7) through the prefill that
    builds the state and the decode steps: each head against the oracle with its own."""
    w = synth.Workload(batch=2, H=6, N=1400, d=64, dtype="f32", seed=93, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    sig = [1.5 + 2.0 * h for h in range(w.H)]
    lam = [0.2 + 0.3 * h for h in range(w.H)]
    N0, T = 1000, 400
    host = pu.inputs(w)
    out, sel, _ = run_stream(w, host, p, N0, T, sigma=sig, lam=lam)
    skipped = checked = 0
    for b in range(w.batch):
        for h in range(w.H):
            op = pu.oracle_params(p, sig[h], lam[h])
            x = tuple(synth.to_f64(host[t][b, h], w.dtype) for t in "qkv")
            ref = pu.attach(oracle.head(*x, None, op, N0, N0 + T), x + (None,), op)
            c, s_ = pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, i_lo=N0, what=f"decode b{b} h{h}")
            checked += c
            skipped += s_
    assert skipped <= 0.01 * (checked + skipped)
