"""GPU tests of fs_attention_decode, the whole attention decode step in one launch
(FreeSolo, Sec. 3.1, Eq. 2: out = o_sr + alpha_h o_lr, with the long-range step of
Sec. 3.3 "Inference" / App. C "Bounded cache" and the local step of Sec. 3.2).

* Against the two separate calls it fuses (fs_longrange_decode, then
  fs_local_decode with its output as o_lr): outputs, selections and both final
  states bitwise equal, over steps that merge at block starts, complete cells and
  wrap the ring.
* Against the fp64 oracle: the long-range rows (oracle.run) combined by the
  oracle's local branch, as in test_gpu_local_decode's two-call test, with the
  rules of tests/parity_utils.py.
* Foreign states, graph replay.
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


def build_states(w, host, p, N0, win):
    """Long-range state from a state-only prefill of the first N0 tokens, local state
    from the same tokens."""
    dt = torch_dtype(w.dtype)
    dk, dv = (pu.to_device(np.ascontiguousarray(host[x][:, :, :N0]), w.dtype) for x in "kv")
    lr = fsl.new_state(w.batch, w.H, w.d, dt, p)
    lr.zero_()
    if N0 > 0:
        fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=lr)
    else:
        fsl.fs_decode_state_init(lr, w.batch, w.H, w.d, dt, p)
    loc = fsl.new_local_state(w.batch, w.H, w.d, dt, w=win)
    loc.zero_()
    fsl.fs_local_state_build(loc, dk, dv, pos=N0, w=win)
    return lr, loc


def run_both(w, p, win, N0, T, gain=None, seed=3):
    """T steps by the two separate calls and by the fused call from equal states.
    Returns the host inputs, both outputs [T, b, H, d], both selections and states."""
    host = pu.inputs(w)
    dt = torch_dtype(w.dtype)
    lr, loc = build_states(w, host, p, N0, win)
    lr2, loc2 = lr.clone(), loc.clone()
    st = {x: steps_of(host[x][:, :, N0:N0 + T], w.dtype) for x in "qkv"}
    alpha = np.random.default_rng(seed).uniform(0.25, 1.75, w.H).astype(np.float32)
    g = None if gain is None else torch.from_numpy(gain).cuda()
    out_a = torch.empty(T, w.batch, w.H, w.d, dtype=dt, device="cuda")
    out_b = torch.empty_like(out_a)
    sel_a = torch.empty(T, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")
    sel_b = torch.empty_like(sel_a)
    print(f"[gpu] attention decode {w} {p} w={win} N0={N0} T={T} gain={gain is not None}", flush=True)
    for t in range(T):
        q, k, v = st["q"][t], st["k"][t], st["v"][t]
        o_lr, _ = fsl.decode(lr, q, k, v, p, gain=g, sel=sel_a[t])
        fsl.fs_local_decode(loc, q, k, v, out_a[t], w=win, alpha=alpha, o_lr=o_lr)
        fsl.fs_attention_decode(lr2, loc2, q, k, v, out_b[t], alpha, sel=sel_b[t], params=p, gain=g, w=win)
    torch.cuda.synchronize()
    return host, alpha, (out_a, sel_a, lr, loc), (out_b, sel_b, lr2, loc2)


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("w,p,win,N0,T,gain", [
    (synth.Workload(batch=2, H=2, N=1100, d=128, dtype="bf16", seed=601, needle_frac=0.005), fsl.Params(), 512,
     1000, 100, False),   # a merge at 1024, cell completions, full window
    (synth.Workload(batch=1, H=3, N=500, d=64, dtype="bf16", seed=602, needle_frac=0.01),
     fsl.Params(K=3, P=6, W=2), 100, 300, 200, True),   # several merges, the ring wraps
    (synth.Workload(batch=2, H=1, N=560, d=128, dtype="f32", seed=603), fsl.Params(K=8), 64, 500, 60, True),
    (synth.Workload(batch=1, H=2, N=168, d=64, dtype="f32", seed=604), fsl.Params(), 0, 128, 40, False),  # w = 0
    (synth.Workload(batch=1, H=2, N=1550, d=128, dtype="bf16", seed=605), fsl.Params(K=1), 1100, 1500, 50,
     False),  # three passes of the ring
    (synth.Workload(batch=1, H=2, N=90, d=128, dtype="bf16", seed=606), fsl.Params(), 512, 0, 90, False),  # empty
], ids=["bf16d128-w512-merge", "bf16d64-w100-wrap", "f32d128-K8", "f32d64-w0", "bf16d128-w1100", "from-empty"])
def test_fused_equals_two_calls(w, p, win, N0, T, gain):
    g = synth.gains(91, w.H, w.d) if gain else None
    _, _, (oa, sa, lra, loca), (ob, sb, lrb, locb) = run_both(w, p, win, N0, T, g)
    assert same_bits(oa, ob), f"outputs differ at {int((oa != ob).sum())} elements"
    assert torch.equal(sa, sb)
    assert torch.equal(lra, lrb), "long-range states differ"
    assert torch.equal(loca, locb), "local states differ"


def test_fused_against_the_oracle():
    """Eq. 2 at decode against the oracle: long-range rows (with near-tie steps read
    out on the GPU's validated selection) combined by the oracle's local branch."""
    w = synth.Workload(batch=2, H=2, N=1400, d=128, dtype="bf16", seed=610, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    N0, T, win = 1000, 120, 512
    host, alpha, _, (out, sels, _, _) = run_both(w, p, win, N0, T)
    got = np.moveaxis(out.float().cpu().numpy(), 0, 2)
    sel = np.moveaxis(sels.cpu().numpy(), 0, 2)
    heads = [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, i_lo=N0, i_hi=N0 + T)
    ties = 0
    for (b, h), ref in refs.items():
        lr_ref, n_tie = pu.lr_reference(sel[b, h], ref, p, N0, f"fused decode b{b} h{h}")
        ties += n_tie
        full = oracle.local(*(synth.to_f64(host[x][b, h], w.dtype) for x in "qkv"), w=win, alpha=float(alpha[h]),
                            o_lr=lr_ref, i_lo=N0, i_hi=N0 + T)
        pu.check_rows(got[b, h], full, w.dtype, f"fused decode output b{b} h{h}", lr_scale=float(alpha[h]))
    assert ties <= 0.01 * len(heads) * T


@pytest.mark.parametrize("which", ["long-range", "local"])
def test_fused_foreign_state(which):
    """A state whose header was not written for this shape: out is NaN, that state is
    left untouched, and the other one advances exactly as the separate call would."""
    w = synth.Workload(batch=1, H=2, N=300, d=64, dtype="bf16", seed=620)
    p = fsl.Params()
    win = 64
    host = pu.inputs(w)
    lr, loc = build_states(w, host, p, 256, win)
    ref_lr, ref_loc = lr.clone(), loc.clone()
    bad = lr if which == "long-range" else loc
    bad[0] ^= 0xFF  # the magic number's first byte
    before = bad.clone()
    q, k, v = (pu.to_device(np.ascontiguousarray(host[x][:, :, 256]), w.dtype) for x in "qkv")
    alpha = np.full(w.H, 0.5, np.float32)
    out = torch.empty(w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    sel = torch.empty(w.batch, w.H, p.K, dtype=torch.int32, device="cuda")
    print(f"[gpu] fused decode with a foreign {which} state", flush=True)
    fsl.fs_attention_decode(lr, loc, q, k, v, out, alpha, sel=sel, params=p, w=win)
    o_ref = torch.empty_like(out)
    o_lr, _ = fsl.decode(ref_lr, q, k, v, p)
    fsl.fs_local_decode(ref_loc, q, k, v, o_ref, w=win, alpha=alpha, o_lr=o_lr)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    assert torch.equal(bad, before)
    if which == "long-range":
        assert (sel == -1).all()
        assert torch.equal(loc, ref_loc)
    else:
        assert torch.equal(lr, ref_lr)


def test_fused_graph_replay():
    """T fused steps captured in one HIP graph and replayed three times, states
    restored in between: every replay equals the eager steps."""
    w = synth.Workload(batch=2, H=2, N=700, d=128, dtype="bf16", seed=630, needle_frac=0.005)
    p = fsl.Params()
    N0, T, win = 600, 40, 512
    host = pu.inputs(w)
    lr, loc = build_states(w, host, p, N0, win)
    lr0, loc0 = lr.clone(), loc.clone()
    st = {x: steps_of(host[x][:, :, N0:N0 + T], w.dtype) for x in "qkv"}
    alpha = np.linspace(0.5, 1.5, w.H).astype(np.float32)
    out = torch.empty(T, w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")

    def run():
        for t in range(T):
            fsl.fs_attention_decode(lr, loc, st["q"][t], st["k"][t], st["v"][t], out[t], alpha, params=p, w=win)

    print(f"[gpu] fused decode graph {w} T={T}", flush=True)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    lr_end, loc_end = lr.clone(), loc.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    lr.copy_(lr0)
    loc.copy_(loc0)
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            run()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(3):
        lr.copy_(lr0)
        loc.copy_(loc0)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert same_bits(out, eager)
        assert torch.equal(lr, lr_end) and torch.equal(loc, loc_end)


def test_fused_decode_shape_sampled():
    """b32 H8 d128 bf16 (the decode workload's grid), w = 512, after an 8,192-token
    prefix: 16 steps, every record against the two separate calls."""
    w = synth.Workload(batch=32, H=8, N=8208, d=128, dtype="bf16", seed=640, needle_frac=0.005)
    _, _, (oa, sa, lra, loca), (ob, sb, lrb, locb) = run_both(w, fsl.Params(), 512, 8192, 16)
    assert same_bits(oa, ob)
    assert torch.equal(sa, sb)
    assert torch.equal(lra, lrb) and torch.equal(loca, locb)
