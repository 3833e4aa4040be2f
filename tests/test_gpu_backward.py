"""GPU parity of the readout backward (fs_readout_backward: FreeSolo Sec. 3.3
"Training", gradients through the selected tokens only, none through the
indices; App. D.4) against the fp64 oracle (oracle.backward) on the same seeded
inputs and the same selections.

Tolerance, per element, from the arithmetic (parity_utils.BWD_REL): the oracle
returns beside each gradient its first-order ERROR SCALE, the sizes of its terms
with every upstream factor's size carried along (so that cancellation in u, r or
the softmax mean widens it where it should).  That scale is a worst-case bound
for a computation whose every step after the softmax rounds to a relative e, so
the bar is e itself:
    |gpu - oracle| <= 2^-16 x error scale   (bf16: split products, 2^-17 per factor),
    |gpu - oracle| <= 2^-19 x error scale   (fp32: the softmax exponent's rounding),
plus 1e-7 x the largest error scale of the tensor.  A CPU test
(test_parity_rules) shows that this bar admits fp32 arithmetic with hi + lo
split operands and rejects the same arithmetic with bf16-only operands.
Elements with no terms at all (a query without a selected cell, a token no query
selected, the tokens past the last complete cell) must be exactly 0.
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


def random_selection(w, p, seed, empty_frac=0.1):
    """Seeded valid selections: for query i, min(K, n) distinct cells among the n
    available to its block (some rows shorter, some empty), -1 padded."""
    rng = np.random.default_rng(seed)
    sel = np.full((w.batch, w.H, w.N, p.K), -1, np.int32)
    cpb = p.B // p.s
    M = w.N // p.s
    for b in range(w.batch):
        for h in range(w.H):
            for i in range(w.N):
                n = min((i // p.B) * cpb, M)
                if n == 0 or rng.random() < empty_frac:
                    continue
                m = min(p.K, n) - (1 if rng.random() < 0.2 and min(p.K, n) > 1 else 0)
                sel[b, h, i, :m] = rng.choice(n, size=m, replace=False)
    return sel


def gpu_backward(w, host, dout, sel, p, gain=None):
    dq_, dk_, dv_ = (pu.to_device(host[x], w.dtype) for x in "qkv")
    g = None if gain is None else torch.from_numpy(gain).cuda()
    do = pu.to_device(dout, w.dtype)
    s = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
    print(f"[gpu] readout backward {w} {p} gain={gain is not None}", flush=True)
    gq, gk, gv, gg, _ = fsl.readout_backward(dq_, dk_, dv_, s, do, g, p)
    torch.cuda.synchronize()
    return gq.cpu().numpy(), gk.cpu().numpy(), gv.cpu().numpy(), (None if gg is None else gg.cpu().numpy())


def check_tensor(got, ref, size, dtype, what):
    """got vs ref element by element against the error scales; exact zero where the scale is 0."""
    got = got.astype(np.float64)
    zero = size == 0
    assert np.all(got[zero] == 0), f"{what}: {int(np.count_nonzero(got[zero]))} nonzero where no term reaches"
    bound = pu.BWD_REL[dtype] * size + pu.BWD_FLOOR * (size.max() if size.size else 0.0)
    err = np.abs(got - ref)
    bad = pu.bwd_beyond_bar(got, ref, size, dtype)
    if bad.any():
        idx = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the bound; worst at {idx}: gpu {got[idx]} "
                             f"oracle {ref[idx]} error scale {size[idx]}")
    nz = size > 0
    return float((err[nz] / size[nz]).max()) if nz.any() else 0.0


def check_backward(w, p, sel, gain=None, heads=None):
    host = pu.inputs(w)
    dout = synth.tensor(w, "dout")
    gq, gk, gv, gg = gpu_backward(w, host, dout, sel, p, gain)
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    op = pu.oracle_params(p)
    dg_ref = {h: np.zeros(w.d) for h in range(w.H)}
    dg_abs = {h: np.zeros(w.d) for h in range(w.H)}
    worst = 0.0
    per = {}
    for b, h in heads:
        x = [synth.to_f64(host[t][b, h], w.dtype) for t in "qkv"]
        gh = None if gain is None else gain[h].astype(np.float64)
        ref = oracle.backward(*x, sel[b, h], synth.to_f64(dout[b, h], w.dtype), gh, op, want_abs=True)
        what = f"{w} b{b} h{h}"
        for name, got in (("dq", gq[b, h]), ("dk", gk[b, h]), ("dv", gv[b, h])):
            e = check_tensor(got, ref[name], ref[name + "_abs"], w.dtype, f"{what} {name}")
            per[name] = max(per.get(name, 0.0), e)
            worst = max(worst, e)
        dg_ref[h] += ref["dg"]
        dg_abs[h] += ref["dg_abs"]
    if gain is not None and len(heads) == w.batch * w.H:
        for h in range(w.H):
            e = check_tensor(gg[h], dg_ref[h], dg_abs[h], w.dtype, f"{w} dgain h{h}")
            per["dgain"] = max(per.get("dgain", 0.0), e)
            worst = max(worst, e)
    print(f"worst error / error scale: {worst:.3g}; " + ", ".join(f"{k} {v:.3g}" for k, v in per.items()))
    return gq, gk, gv, gg


def prefill_selection(w, p, gain=None):
    """The selections the FS-L prefill makes on these inputs (the concentrated pattern
    training sees: many queries of a block share their cells)."""
    host = pu.inputs(w)
    q, k, v = (pu.to_device(host[x], w.dtype) for x in "qkv")
    _, sel, _ = fsl.prefill(q, k, v, p, want_out=False)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


@pytest.mark.parametrize("w,p,how,gain", [
    (synth.Workload(batch=1, H=2, N=4096, d=64, dtype="bf16", seed=501, needle_frac=0.005), fsl.Params(),
     "prefill", True),
    (synth.Workload(batch=1, H=2, N=2500, d=128, dtype="bf16", seed=502, needle_frac=0.01), fsl.Params(),
     "random", False),
    (synth.Workload(batch=2, H=1, N=1100, d=64, dtype="f32", seed=503), fsl.Params(K=8), "random", True),
    (synth.Workload(batch=1, H=2, N=700, d=128, dtype="f32", seed=504, needle_frac=0.01), fsl.Params(K=1),
     "prefill", False),
    (synth.Workload(batch=1, H=2, N=3000, d=128, dtype="bf16", seed=505), fsl.Params(K=6, P=16, W=4),
     "prefill", True),
    (synth.Workload(batch=1, H=2, N=1536, d=64, dtype="bf16", seed=506, needle_frac=0.01),
     fsl.Params(K=3, prune=False), "prefill", False),
], ids=["bf16d64-train-like", "bf16d128-ragged-random", "f32d64-K8-random", "f32d128-K1", "bf16d128-K6-P16",
        "bf16d64-FS-K3"])
def test_readout_backward(w, p, how, gain):
    sel = prefill_selection(w, p) if how == "prefill" else random_selection(w, p, seed=w.seed)
    check_backward(w, p, sel, synth.gains(97, w.H, w.d) if gain else None)


@pytest.mark.parametrize("N", [1, 127, 128, 129, 160, 300])
def test_backward_tiny_and_ragged(N):
    """No cell is available before the second block: every gradient of the first 128
    queries and of their keys is 0; past it the random selections are checked."""
    w = synth.Workload(batch=1, H=2, N=N, d=64, dtype="bf16", seed=520 + N)
    p = fsl.Params()
    sel = random_selection(w, p, seed=N)
    gq, gk, gv, gg = check_backward(w, p, sel, synth.gains(98, 2, 64))
    assert np.all(gq[:, :, :min(N, 128)] == 0)


def test_backward_empty_selection():
    w = synth.Workload(batch=1, H=2, N=1000, d=128, dtype="bf16", seed=530)
    p = fsl.Params(K=3)
    sel = np.full((1, 2, 1000, 3), -1, np.int32)
    gq, gk, gv, gg = gpu_backward(w, pu.inputs(w), synth.tensor(w, "dout"), sel, p, synth.gains(99, 2, 128))
    assert not gq.any() and not gk.any() and not gv.any() and not gg.any()


def test_backward_one_cell_for_every_query():
    """Every query from block 1 on selects cell 0 (and cells of its own choice): cell 0's
    query list (3968 queries) spans two windows of the key side's list."""
    w = synth.Workload(batch=1, H=1, N=4096, d=128, dtype="bf16", seed=540, needle_frac=0.005)
    p = fsl.Params(K=4)
    sel = random_selection(w, p, seed=540, empty_frac=0.0)
    for i in range(128, w.N):
        row = [c for c in sel[0, 0, i] if c > 0][:3]
        sel[0, 0, i] = [0] + row + [-1] * (3 - len(row))
    check_backward(w, p, sel)


def test_backward_training_shape_sampled():
    """b16 H16 d64 N4096 bf16 with the FS-L prefill's selections (one GPU's share of the
    pages' 524,288-token training step): the whole batch on the GPU, every gradient of
    two sampled (sequence, head) pairs against the oracle."""
    w = synth.WORKLOADS["train_4k"]
    p = fsl.Params()
    sel = prefill_selection(w, p)
    check_backward(w, p, sel, synth.gains(96, w.H, w.d), heads=[(0, 5), (15, 11)])


def test_backward_longest_sequence_sampled():
    """N = 65,536, the longest the backward accepts: one head, every gradient checked."""
    w = synth.Workload(batch=1, H=1, N=65536, d=64, dtype="bf16", seed=550, needle_frac=0.005)
    p = fsl.Params()
    sel = prefill_selection(w, p)
    check_backward(w, p, sel)


def test_backward_deterministic():
    w = synth.Workload(batch=2, H=2, N=2048, d=128, dtype="bf16", seed=560, needle_frac=0.005)
    p = fsl.Params()
    sel = prefill_selection(w, p)
    host = pu.inputs(w)
    dout = synth.tensor(w, "dout")
    g = synth.gains(95, 2, 128)
    a = gpu_backward(w, host, dout, sel, p, g)
    b = gpu_backward(w, host, dout, sel, p, g)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
