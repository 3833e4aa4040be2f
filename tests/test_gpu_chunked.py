"""GPU parity of chunked prefill into a decode state (fs_longrange_prefill_chunk;
FreeSolo App. C "Bounded cache": prefill in fixed-size chunks, the page's 2048
tokens, with the retention update at every block boundary) and of multi-layer
decode under one HIP graph.

The page defines prefill and decode as one causal operator (Sec. 3.3
"Inference"), so the reference for every chunk position is the oracle's output
at that position over the whole sequence; see tests/parity_utils.py for the
rules.  A chunk must also agree bitwise with itself split at any point.  bf16
chunks are computed block by block with the whole-prompt prefill's arithmetic,
so they agree with it bitwise; fp32 chunks are n decode steps in one launch,
bitwise n single steps.
"""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import synth
from tests import parity_utils as pu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fsl.lib()


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def rows(host, x, lo, hi, dtype):
    return pu.to_device(np.ascontiguousarray(host[x][:, :, lo:hi]), dtype)


def empty_state(w, p):
    st = fsl.new_state(w.batch, w.H, w.d, tdtype(w), p)
    st.fill_(0x5A)  # whatever the buffer held: the init writes what a state needs
    fsl.fs_decode_state_init(st, w.batch, w.H, w.d, tdtype(w), p)
    return st


def run_chunks(w, host, p, state, lo, bounds, sigma=4.0, lam=1.0, gain=None):
    """Feed positions lo .. bounds[-1] in chunks ending at each bound; returns (out, sel) [b, H, n, ...]."""
    outs, sels = [], []
    g = None if gain is None else torch.from_numpy(gain).cuda()
    for hi in bounds:
        print(f"[gpu] chunk {w} {p} [{lo}, {hi})", flush=True)
        q, k, v = (rows(host, x, lo, hi, w.dtype) for x in "qkv")
        o, s = fsl.prefill_chunk(state, q, k, v, p, sigma=sigma, lam=lam, gain=g)
        outs.append(o)
        sels.append(s)
        lo = hi
    torch.cuda.synchronize()
    return torch.cat(outs, dim=2).float().cpu().numpy(), torch.cat(sels, dim=2).cpu().numpy()


@pytest.mark.parametrize("w,p,bounds,extra", [
    # a whole prompt from an empty state, in chunks of 2048 and a ragged last one
    (synth.Workload(batch=2, H=2, N=5000, d=128, dtype="bf16", seed=501, needle_frac=0.005), fsl.Params(),
     [2048, 4096, 5000], {}),
    (synth.Workload(batch=1, H=3, N=3000, d=64, dtype="f32", seed=502, needle_frac=0.01), fsl.Params(P=6, W=2),
     [1000, 1001, 2048, 3000], {}),
    (synth.Workload(batch=1, H=2, N=2500, d=128, dtype="bf16", seed=503, needle_frac=0.01), fsl.Params(P=10, W=3, K=8),
     [2048, 2500], {"gain": True}),
    (synth.Workload(batch=1, H=2, N=1500, d=64, dtype="bf16", seed=504), fsl.Params(P=5, W=2), [700, 1500],
     {"lam": 0.0}),
], ids=["bf16d128-2048x2+904", "f32d64-ragged-chunks", "bf16-K8-gain", "lam0"])
def test_chunked_prompt_from_empty_state(w, p, bounds, extra):
    host = pu.inputs(w)
    gain = synth.gains(95, w.H, w.d) if extra.get("gain") else None
    lam = extra.get("lam", 1.0)
    st = empty_state(w, p)
    out, sel = run_chunks(w, host, p, st, 0, bounds, lam=lam, gain=gain)
    heads = [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, 4.0, lam, gain)
    exact = ties = 0
    for (b, h), ref in refs.items():
        c, t = pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, what=f"chunked b{b} h{h}")
        exact += c
        ties += t
    print(f"checked {exact} queries exactly, {ties} near-ties validated")
    assert ties <= 0.01 * (exact + ties)
    # the whole-prompt prefill selects the same cells (the same causal operator)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    _, sel_pre, _ = fsl.prefill(dq, dk, dv, p, lam=lam)
    sel_pre = sel_pre.cpu().numpy()
    for (b, h), ref in refs.items():
        ok = ~pu.excluded_queries(ref, p, 0, w.N)
        np.testing.assert_array_equal(sel[b, h][ok], sel_pre[b, h][ok])


@pytest.mark.parametrize("w,p", [
    (synth.Workload(batch=2, H=2, N=2600, d=128, dtype="bf16", seed=505, needle_frac=0.01), fsl.Params(P=8, W=2)),
    (synth.Workload(batch=1, H=3, N=1900, d=64, dtype="bf16", seed=507, needle_frac=0.01), fsl.Params(K=6)),
    (synth.Workload(batch=2, H=2, N=2600, d=128, dtype="f32", seed=508, needle_frac=0.01), fsl.Params(P=8, W=2)),
], ids=["bf16d128", "bf16d64-K6", "f32d128"])
def test_chunk_split_anywhere_and_against_prefill(w, p):
    """The same tokens in one chunk or split into two at any point: bitwise the same
    outputs, selections and final state.  bf16 chunks run block by block with the
    fused prefill's arithmetic, so they are bitwise the whole-prompt prefill's rows;
    fp32 chunks are single decode steps, so they are bitwise n single steps."""
    host = pu.inputs(w)
    N0, n = 1000, w.N - 1000 - 300  # a state from a prefill, then positions crossing several block boundaries
    dk, dv = (rows(host, x, 0, N0, w.dtype) for x in "kv")
    base = fsl.new_state(w.batch, w.H, w.d, tdtype(w), p)
    base.fill_(0x33)
    fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=base)
    s1, s2, s3 = base.clone(), base.clone(), base.clone()
    o1, c1 = run_chunks(w, host, p, s1, N0, [N0 + n])
    o3, c3 = run_chunks(w, host, p, s3, N0, [N0 + 437, N0 + n])
    np.testing.assert_array_equal(c1, c3)
    np.testing.assert_array_equal(o1, o3)
    assert torch.equal(s1, s3)
    if w.dtype == "bf16":
        dq, dk2, dv2 = (rows(host, x, 0, N0 + n, w.dtype) for x in "qkv")
        print(f"[gpu] whole-prompt prefill {w}", flush=True)
        o_pre, c_pre, _ = fsl.prefill(dq, dk2, dv2, p)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(c1, c_pre[:, :, N0:].cpu().numpy())
        np.testing.assert_array_equal(o1, o_pre[:, :, N0:].float().cpu().numpy())
        return
    steps = {x: pu.to_device(np.ascontiguousarray(np.moveaxis(host[x][:, :, N0:N0 + n], 2, 0)), w.dtype) for x in "qkv"}
    outs = torch.empty(n, w.batch, w.H, w.d, dtype=tdtype(w), device="cuda")
    sels = torch.empty(n, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")
    print("[gpu] single steps", flush=True)
    for t in range(n):
        fsl.decode(s2, steps["q"][t], steps["k"][t], steps["v"][t], p, out=outs[t], sel=sels[t])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c1, np.moveaxis(sels.cpu().numpy(), 0, 2))
    np.testing.assert_array_equal(o1, np.moveaxis(outs.float().cpu().numpy(), 0, 2))
    assert torch.equal(s1, s2)


def state_summaries(st, w):
    """(cell ids [b H, S], fp32 mean keys [b H, S, d], norms [b H, S]) of a decode-state
    buffer, read in the record layout fs_decode_state_bytes sizes: a 256-byte header
    (n_slots at byte 40, the record size at byte 48), then per (sequence, head) a
    32-byte meta block and the slot tables (positions in A, cell ids, flags, a_c,
    mean keys), each starting on a 256-byte boundary."""
    raw = st.cpu().numpy()
    S = int(raw[40:44].view(np.int32)[0])
    rec = int(raw[48:56].view(np.int64)[0])
    al = lambda x: (x + 255) // 256 * 256
    off_cell = al(32) + al(4 * S)
    off_a = off_cell + 2 * al(4 * S)
    off_kbar = off_a + al(4 * S)
    n = w.batch * w.H
    cells = np.stack([raw[256 + r * rec + off_cell:][:4 * S].view(np.int32) for r in range(n)])
    a = np.stack([raw[256 + r * rec + off_a:][:4 * S].view(np.float32) for r in range(n)])
    kbar = np.stack([raw[256 + r * rec + off_kbar:][:4 * S * w.d].view(np.float32).reshape(S, w.d) for r in range(n)])
    return cells, kbar, a


def test_chunks_from_empty_state_equal_prefill_bitwise():
    """bf16: a whole prompt fed from an empty state in chunks of 2048 (and a ragged
    last one, and chunks ending mid-cell) gives bitwise the whole-prompt prefill's
    output rows and selections, and every complete cell the state holds has bitwise
    the summary pass's mean key and norm (Eq. 5)."""
    w = synth.Workload(batch=2, H=3, N=5000, d=128, dtype="bf16", seed=509, needle_frac=0.005)
    p = fsl.Params()
    host = pu.inputs(w)
    st = empty_state(w, p)
    o, c = run_chunks(w, host, p, st, 0, [2048, 2049, 3000, 4096, 4113, 5000])
    dq, dk, dv = (rows(host, x, 0, w.N, w.dtype) for x in "qkv")
    o_pre, c_pre, _ = fsl.prefill(dq, dk, dv, p)
    M = w.N // p.s
    kbar_ref = torch.empty(w.batch, w.H, M, w.d, dtype=torch.float32, device="cuda")
    a_ref = torch.empty(w.batch, w.H, M, dtype=torch.float32, device="cuda")
    fsl.fs_cell_summaries(dk, kbar_ref, a_ref, p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c, c_pre.cpu().numpy())
    np.testing.assert_array_equal(o, o_pre.float().cpu().numpy())
    cells, kbar, a = state_summaries(st, w)
    kbar_ref = kbar_ref.reshape(w.batch * w.H, M, w.d).cpu().numpy()
    a_ref = a_ref.reshape(w.batch * w.H, M).cpu().numpy()
    checked = 0
    for r in range(w.batch * w.H):
        for x, cell in enumerate(cells[r]):
            if 0 <= cell < M:
                assert np.array_equal(kbar[r, x].view(np.uint32), kbar_ref[r, cell].view(np.uint32)), (r, cell)
                assert a[r, x].view(np.uint32) == a_ref[r, cell].view(np.uint32), (r, cell)
                checked += 1
    assert checked >= w.batch * w.H * p.P


def test_chunked_prefill_then_decode_equals_prefill_then_decode():
    """A state reached by chunks from an empty state decodes bitwise like the state the
    whole-prompt prefill builds (same retained cells and summaries; slots may differ)."""
    w = synth.Workload(batch=1, H=4, N=4300, d=128, dtype="bf16", seed=506, needle_frac=0.005)
    p = fsl.Params()
    host = pu.inputs(w)
    N0 = 4096
    st_c = empty_state(w, p)
    run_chunks(w, host, p, st_c, 0, [2048, N0])
    st_p = fsl.new_state(w.batch, w.H, w.d, torch.bfloat16, p)
    dk, dv = (rows(host, x, 0, N0, w.dtype) for x in "kv")
    fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=st_p)
    oc, cc = run_chunks(w, host, p, st_c, N0, [w.N])
    op, cp = run_chunks(w, host, p, st_p, N0, [w.N])
    np.testing.assert_array_equal(cc, cp)
    np.testing.assert_array_equal(oc, op)
    refs = pu.run_oracle(w, host, p, [(0, 0), (0, 3)], i_lo=N0, i_hi=w.N)
    for (b, h), ref in refs.items():
        pu.compare_head(cc[b, h], oc[b, h], ref, p, w.dtype, i_lo=N0, what=f"after chunks b{b} h{h}")


def test_chunk_decode_shape_sampled():
    """The decode workload's shape per sequence (H=8, d=128, bf16, a 262,144-token prefix)
    for two sequences, then one 2048-token chunk (the page's chunk size): sampled heads of
    every chunk position against the oracle."""
    w0 = synth.WORKLOADS["decode_256k"]
    N0, n = 262144, 2048
    w = synth.Workload(batch=2, H=8, N=N0 + n, d=w0.d, dtype=w0.dtype, seed=w0.seed, needle_frac=w0.needle_frac)
    p = fsl.Params()
    host = pu.inputs(w)
    st = fsl.new_state(w.batch, w.H, w.d, torch.bfloat16, p)
    dk, dv = (rows(host, x, 0, N0, w.dtype) for x in "kv")
    print(f"[gpu] prefix prefill {w}", flush=True)
    fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=st)
    del dk, dv
    out, sel = run_chunks(w, host, p, st, N0, [N0 + n])
    refs = pu.run_oracle(w, host, p, [(0, 2), (1, 5)], i_lo=N0, i_hi=N0 + n)
    for (b, h), ref in refs.items():
        pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, i_lo=N0, what=f"2048-token chunk b{b} h{h}")


def test_chunk_rejects_foreign_state():
    p = fsl.Params()
    b, H, d, n = 2, 3, 64, 40
    st = fsl.new_state(b, H, d, torch.float32, p)
    st.zero_()
    q = torch.randn(b, H, n, d, device="cuda")
    o, s = fsl.prefill_chunk(st, q, q, q, p)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and (s == -1).all()
    assert int(st.count_nonzero()) == 0


def test_multi_layer_decode_graph():
    """L = 4 layers' decode steps (each layer its own state, its own q/k/v), 200 steps
    captured as one HIP graph: every replay (state restored, eager work in between) gives
    bitwise the eager results."""
    L_, T = 4, 200
    w = synth.Workload(batch=2, H=4, N=1200 + T, d=128, dtype="bf16", seed=507, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    N0 = 1200
    states, snaps, steps = [], [], []
    for layer in range(L_):
        wl = synth.Workload(batch=w.batch, H=w.H, N=w.N, d=w.d, dtype=w.dtype, seed=w.seed + layer,
                            needle_frac=w.needle_frac)
        host = pu.inputs(wl)
        st = fsl.new_state(w.batch, w.H, w.d, torch.bfloat16, p)
        dk, dv = (rows(host, x, 0, N0, w.dtype) for x in "kv")
        fsl.prefill(None, dk, dv, p, want_out=False, want_sel=False, state=st)
        states.append(st)
        snaps.append(st.clone())
        steps.append({x: pu.to_device(np.ascontiguousarray(np.moveaxis(host[x][:, :, N0:], 2, 0)), w.dtype)
                      for x in "qkv"})
    outs = torch.empty(L_, T, w.batch, w.H, w.d, dtype=torch.bfloat16, device="cuda")
    sels = torch.empty(L_, T, w.batch, w.H, p.K, dtype=torch.int32, device="cuda")

    def run_all():
        for t in range(T):
            for layer in range(L_):
                fsl.decode(states[layer], steps[layer]["q"][t], steps[layer]["k"][t], steps[layer]["v"][t], p,
                           out=outs[layer, t], sel=sels[layer, t])

    print("[gpu] multi-layer graph", flush=True)
    run_all()
    torch.cuda.synchronize()
    ref_o, ref_s = outs.clone(), sels.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for layer in range(L_):
            states[layer].copy_(snaps[layer])
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for layer in range(L_):
            states[layer].copy_(snaps[layer])
        outs.zero_()
        sels.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sels, ref_s), f"replay {rep}: selections differ"
        assert torch.equal(outs.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: outputs differ"
