"""GPU parity: the gfx950 path through the C ABI against the fp64 oracle, on the
same seeded inputs.  Selections must match exactly (near-ties validated and
counted), outputs within the stated tolerances; see tests/parity_utils.py for the
rules."""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import oracle
import synth
from tests import parity_utils as pu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def gpu_available():
    return torch.cuda.is_available()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not gpu_available():
        pytest.skip("needs a GPU")
    fsl.lib()


def run_prefill(w, host, p, sigma=4.0, lam=1.0, gain=None):
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    g = None if gain is None else torch.from_numpy(gain).cuda()
    print(f"[gpu] prefill {w} {p}", flush=True)
    out, sel, _ = fsl.prefill(dq, dk, dv, p, sigma=sigma, lam=lam, gain=g)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), sel.cpu().numpy()


def check(w, p, heads=None, sigma=4.0, lam=1.0, gain=None, max_skip_frac=0.01):
    host = pu.inputs(w)
    out, sel = run_prefill(w, host, p, sigma, lam, gain)
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, sigma, lam, gain)
    checked = skipped = 0
    for (b, h), ref in refs.items():
        c, s = pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, what=f"{w.name or w} b{b} h{h}")
        checked += c
        skipped += s
    print(f"checked {checked} queries exactly, {skipped} near-ties validated")
    assert skipped <= max_skip_frac * (checked + skipped)
    return out, sel


# ---------------------------------------------------------------- summaries ----

@pytest.mark.parametrize("w", [
    synth.WORKLOADS["small_fs_equiv"],
    synth.WORKLOADS["prefill_4k"],
    synth.Workload(batch=2, H=3, N=1000, d=128, dtype="bf16", seed=21, needle_frac=0.01),
    synth.Workload(batch=1, H=2, N=777, d=64, dtype="bf16", seed=22),
    synth.Workload(batch=1, H=1, N=31, d=128, dtype="f32", seed=23),
], ids=lambda w: f"b{w.batch}H{w.H}N{w.N}d{w.d}{w.dtype}")
def test_cell_summaries(w):
    host = pu.inputs(w)
    k = pu.to_device(host["k"], w.dtype)
    M = w.N // 32
    kbar = torch.empty(w.batch, w.H, M, w.d, dtype=torch.float32, device="cuda")
    a = torch.empty(w.batch, w.H, M, dtype=torch.float32, device="cuda")
    ks = torch.full((w.batch, w.H, M, 3, w.d), -1, dtype=torch.int16, device="cuda")
    kn = torch.full((w.batch, w.H, M), -1.0, dtype=torch.float32, device="cuda")
    print(f"[gpu] summaries {w}", flush=True)
    fsl.fs_cell_summaries(k, kbar, a, kbar_split=ks, kbar_norm=kn)
    torch.cuda.synchronize()
    kbar, a, ks, kn = kbar.cpu().numpy(), a.cpu().numpy(), ks.cpu().numpy().view(np.uint16), kn.cpu().numpy()
    # the norm of the stored fp32 mean, summed in fp64 and rounded once
    np.testing.assert_allclose(kn, np.sqrt((kbar.astype(np.float64) ** 2).sum(-1)), rtol=1.2e-7, atol=0)
    import oracle
    for b in range(w.batch):
        for h in range(w.H):
            rk, ra = oracle.cell_summaries(synth.to_f64(host["k"][b, h], w.dtype))
            # fp64 sums rounded once: the mean is the correctly rounded fp32 of the exact mean
            np.testing.assert_array_equal(kbar[b, h], rk.astype(np.float32))
            np.testing.assert_allclose(a[b, h], ra, rtol=1.2e-7, atol=0)
    if w.dtype == "bf16":
        # the three bf16 parts: hi = bf16(kbar), mid = bf16(kbar - hi), lo = bf16(kbar - hi - mid), nearest-even
        def rne(x):
            u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
            return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

        def widen(hb):
            return (hb.astype(np.uint32) << 16).view(np.float32)

        hi = rne(kbar)
        r1 = (kbar - widen(hi)).astype(np.float32)
        mid = rne(r1)
        lo = rne((r1 - widen(mid)).astype(np.float32))
        np.testing.assert_array_equal(ks[..., 0, :], hi)
        np.testing.assert_array_equal(ks[..., 1, :], mid)
        np.testing.assert_array_equal(ks[..., 2, :], lo)
    else:
        assert np.all(ks == 0xFFFF)  # not written for fp32 shapes


# ------------------------------------------------------------------ pruning ----

@pytest.mark.parametrize("w,P,W", [
    (synth.WORKLOADS["prefill_4k"], 64, 8),
    (synth.Workload(batch=2, H=2, N=5000, d=64, dtype="f32", seed=31, needle_frac=0.01), 5, 3),
    (synth.Workload(batch=1, H=2, N=3000, d=128, dtype="bf16", seed=32), 0, 4),
    (synth.Workload(batch=1, H=2, N=3000, d=128, dtype="bf16", seed=33), 7, 0),
    # heads of up to 4096 cells are ranked once and filtered per block; longer ones take the other kernels
    (synth.Workload(batch=1, H=1, N=4096 * 32 + 31, d=64, dtype="bf16", seed=34, needle_frac=0.005), 64, 8),
    (synth.Workload(batch=1, H=1, N=4100 * 32, d=64, dtype="bf16", seed=35, needle_frac=0.005), 64, 8),
], ids=["cfg4k", "P5W3", "P0W4", "P7W0", "M4096-ranked", "M4100-per-block"])
def test_prune_retained(w, P, W):
    p = fsl.Params(P=P, W=W)
    host = pu.inputs(w)
    k = pu.to_device(host["k"], w.dtype)
    M, NB, cap = w.N // 32, (w.N + 127) // 128, max(1, P + W)
    kbar = torch.empty(w.batch, w.H, M, w.d, dtype=torch.float32, device="cuda")
    a = torch.empty(w.batch, w.H, M, dtype=torch.float32, device="cuda")
    fsl.fs_cell_summaries(k, kbar, a, p)
    sh = fsl.shape_of(k)
    ws = torch.empty(fsl.fs_prune_workspace_bytes(sh, p), dtype=torch.uint8, device="cuda")
    ret = torch.empty(w.batch, w.H, NB, cap, dtype=torch.int32, device="cuda")
    nret = torch.empty(w.batch, w.H, NB, dtype=torch.int32, device="cuda")
    print(f"[gpu] prune {w} P={P} W={W}", flush=True)
    fsl.fs_prune_retained(sh, a, ret, nret, ws, p)
    torch.cuda.synchronize()
    ret, nret, a_gpu = ret.cpu().numpy(), nret.cpu().numpy(), a.cpu().numpy()
    import oracle
    op = pu.oracle_params(p)
    ties = blocks = 0
    for b in range(w.batch):
        for h in range(w.H):
            ref = oracle.head(None, synth.to_f64(host["k"][b, h], w.dtype), None, prm=op, want_out=False)
            for beta in range(NB):
                blocks += 1
                n = nret[b, h, beta]
                row = ret[b, h, beta, :n]
                # listed in priority order (a desc, id asc) of the norms the GPU computed
                key = [(-a_gpu[b, h, c], c) for c in row]
                assert key == sorted(key), (b, h, beta)
                assert np.all(ret[b, h, beta, n:] == -1)
                if ref["gap_p"][beta] < pu.NEAR_TIE:
                    # several retained sets are correct: check that this is one of them
                    ties += 1
                    pu.check_retained_valid(row, ref["a"], oracle.available_count(128 * beta, 32), P, W)
                    continue
                assert n == ref["n_ret"][beta], (b, h, beta)
                np.testing.assert_array_equal(np.sort(row), ref["retained"][beta, :n])
    print(f"checked {blocks} blocks, {ties} at a TopP near-tie validated")
    assert ties <= 0.01 * blocks


# ------------------------------------------------------------ whole prefill ----

def test_config_small_fs_equivalent():
    """1024 tokens, 32 cells: pruning never binds, so FS-L equals FS (both checked)."""
    w = synth.WORKLOADS["small_fs_equiv"]
    _, sel_l = check(w, fsl.Params(prune=True))
    _, sel_f = check(w, fsl.Params(prune=False))
    np.testing.assert_array_equal(sel_l, sel_f)


def test_config_4k_pruning_active():
    check(synth.WORKLOADS["prefill_4k"], fsl.Params())


@pytest.mark.parametrize("w,p,extra", [
    (synth.Workload(batch=2, H=2, N=2000, d=128, dtype="bf16", seed=41, needle_frac=0.005), fsl.Params(), {}),
    (synth.Workload(batch=1, H=3, N=1500, d=64, dtype="bf16", seed=42, needle_frac=0.01), fsl.Params(P=6, W=2), {}),
    (synth.Workload(batch=1, H=2, N=2100, d=128, dtype="f32", seed=43, needle_frac=0.01), fsl.Params(P=10, W=4), {}),
    (synth.Workload(batch=1, H=2, N=1300, d=64, dtype="f32", seed=44), fsl.Params(prune=False), {}),
    (synth.Workload(batch=1, H=2, N=1300, d=128, dtype="bf16", seed=45, needle_frac=0.01), fsl.Params(prune=False), {}),
    (synth.Workload(batch=1, H=2, N=1024, d=64, dtype="f32", seed=46), fsl.Params(K=1), {}),
    (synth.Workload(batch=1, H=2, N=1024, d=128, dtype="bf16", seed=47), fsl.Params(K=3, P=5, W=1), {}),
    (synth.Workload(batch=1, H=2, N=1024, d=64, dtype="bf16", seed=48), fsl.Params(K=8, P=9, W=3), {}),
    (synth.Workload(batch=1, H=2, N=1024, d=64, dtype="f32", seed=49), fsl.Params(P=0, W=0), {}),
    (synth.Workload(batch=1, H=2, N=1024, d=64, dtype="f32", seed=50), fsl.Params(P=0, W=2, K=4), {}),
    (synth.Workload(batch=1, H=2, N=1200, d=64, dtype="f32", seed=51, needle_frac=0.01), fsl.Params(), {"lam": 0.0}),
    (synth.Workload(batch=1, H=2, N=1200, d=128, dtype="bf16", seed=52, needle_frac=0.01), fsl.Params(),
     {"lam": 0.0}),
    (synth.Workload(batch=1, H=2, N=1200, d=64, dtype="f32", seed=53), fsl.Params(), {"sigma": 40.0, "lam": 0.3}),
    (synth.Workload(batch=1, H=4, N=1100, d=128, dtype="bf16", seed=54, needle_frac=0.01), fsl.Params(P=12, W=3),
     {"gain": True}),
], ids=["bf16d128", "bf16d64P6", "f32d128P10", "FSf32", "FSbf16", "K1", "K3", "K8", "P0W0", "P0W2", "lam0f32",
        "lam0bf16", "sigma40", "gain"])
def test_prefill_variants(w, p, extra):
    gain = synth.gains(99, w.H, w.d) if extra.get("gain") else None
    check(w, p, sigma=extra.get("sigma", 4.0), lam=extra.get("lam", 1.0), gain=gain)


@pytest.mark.parametrize("N", [1, 31, 32, 127, 128, 129, 160, 1023])
def test_ragged_and_tiny_lengths(N):
    w = synth.Workload(batch=1, H=2, N=N, d=64, dtype="bf16", seed=60 + N, needle_frac=0.02)
    out, sel = check(w, fsl.Params(P=3, W=1))
    assert np.all(sel[:, :, :min(N, 128)] == -1) and np.all(out[:, :, :min(N, 128)] == 0)


def test_deterministic():
    w = synth.Workload(batch=1, H=2, N=2048, d=128, dtype="bf16", seed=70, needle_frac=0.005)
    host = pu.inputs(w)
    o1, s1 = run_prefill(w, host, fsl.Params())
    o2, s2 = run_prefill(w, host, fsl.Params())
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(o1, o2)


# --------------------------------------------------- full-size, sampled heads ----

def test_headline_16k_sampled_heads():
    """b4 H16 d128 N16384 bf16: the whole batch on the GPU, every query of sampled
    (sequence, head) pairs against the oracle."""
    w = synth.WORKLOADS["prefill_16k"]
    check(w, fsl.Params(), heads=[(0, 0), (1, 5), (2, 10), (3, 15)])


def test_fs_32k_sampled():
    """FS (no pruning), b1 H16 d128 N32768 bf16: up to 1020 cells scored per query."""
    w = synth.WORKLOADS["fs_32k"]
    check(w, fsl.Params(prune=False), heads=[(0, 3), (0, 12)])


def test_maximum_length_sampled_blocks():
    """N = 2^22, the longest sequence the ABI accepts: 131,072 cells per head, so the
    retained sets take the per-block pruning path.  The whole sequence runs on the GPU;
    the queries of an early, a middle and the last block are compared with the oracle."""
    w = synth.Workload(batch=1, H=1, N=1 << 22, d=64, dtype="bf16", seed=80, needle_frac=0.001)
    p = fsl.Params()
    host = pu.inputs(w)
    out, sel = run_prefill(w, host, p)
    qf, kf, vf = (synth.to_f64(host[x][0, 0], w.dtype) for x in "qkv")
    del host
    checked = skipped = 0
    for lo in (128 * 40, (w.N // 2) // 128 * 128, w.N - 128):
        op = pu.oracle_params(p)
        ref = pu.attach(oracle.head(qf, kf, vf, None, op, lo, lo + 128), (qf, kf, vf, None), op)
        c, s = pu.compare_head(sel[0, 0, lo:lo + 128], out[0, 0, lo:lo + 128], ref, p, w.dtype, i_lo=lo,
                               what=f"N=2^22 block {lo // 128}")
        checked += c
        skipped += s
    print(f"checked {checked} queries exactly, {skipped} near-ties validated")
    assert skipped <= 0.01 * (checked + skipped)


def test_per_head_constants_at_max_heads():
    """H = 128, the most heads accepted, each with its own sigma_h and lambda_h (Eq. 7):
    sampled heads against the oracle with that head's constants."""
    w = synth.Workload(batch=1, H=128, N=700, d=64, dtype="f32", seed=81, needle_frac=0.01)
    p = fsl.Params(P=6, W=2)
    sig = [2.0 + h / 16.0 for h in range(w.H)]
    lam = [0.25 + h / 64.0 for h in range(w.H)]
    host = pu.inputs(w)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    print(f"[gpu] per-head constants {w}", flush=True)
    out, sel, _ = fsl.prefill(dq, dk, dv, p, sigma=sig, lam=lam)
    torch.cuda.synchronize()
    out, sel = out.float().cpu().numpy(), sel.cpu().numpy()
    for h in (0, 1, 63, 127):
        op = pu.oracle_params(p, sig[h], lam[h])
        x = tuple(synth.to_f64(host[t][0, h], w.dtype) for t in "qkv")
        ref = pu.attach(oracle.head(*x, None, op), x + (None,), op)
        pu.compare_head(sel[0, h], out[0, h], ref, p, w.dtype, what=f"H=128 head {h}")


def test_largest_grid_sampled_heads():
    """batch * H = 65,408 (b511 H128), close to the 65,535 the ABI accepts, N = 160 (one
    routed block per head): the long-range prefill and the local branch over every head,
    sampled heads against the oracle."""
    w = synth.Workload(batch=511, H=128, N=160, d=64, dtype="bf16", seed=82, needle_frac=0.02)
    p = fsl.Params()
    host = pu.inputs(w)
    out, sel = run_prefill(w, host, p)
    dq, dk, dv = (pu.to_device(host[x], w.dtype) for x in "qkv")
    loc = fsl.local(dq, dk, dv, w=64).float().cpu().numpy()
    heads = [(0, 0), (255, 64), (510, 127)]
    for (b, h), ref in pu.run_oracle(w, host, p, heads).items():
        pu.compare_head(sel[b, h], out[b, h], ref, p, w.dtype, what=f"b{b} h{h}")
        lref = oracle.local(*(synth.to_f64(host[x][b, h], w.dtype) for x in "qkv"), w=64)
        pu.check_rows(loc[b, h], lref, w.dtype, f"local b{b} h{h}")


@pytest.mark.parametrize("P,W", [(240, 16), (300, 20)], ids=["cap256-single-kernel", "cap320-two-kernels"])
def test_large_retained_sets(P, W):
    """Retained sets at the single-kernel limit (P + W = 256) and past it (the
    prefill then scores and reads out in two kernels), bf16 d128 N8192."""
    w = synth.Workload(batch=1, H=2, N=8192, d=128, dtype="bf16", seed=79, needle_frac=0.01)
    check(w, fsl.Params(P=P, W=W))


def test_score_with_precomputed_split_matches():
    """fs_score_select with the bf16 parts from fs_cell_summaries selects exactly what it
    selects when it splits the fp32 means itself (same operands on the matrix cores)."""
    w = synth.Workload(batch=2, H=2, N=3000, d=128, dtype="bf16", seed=71, needle_frac=0.01)
    p = fsl.Params()
    host = pu.inputs(w)
    q, k = (pu.to_device(host[x], w.dtype) for x in "qk")
    M, NB = w.N // 32, (w.N + 127) // 128
    kbar = torch.empty(w.batch, w.H, M, w.d, dtype=torch.float32, device="cuda")
    a = torch.empty(w.batch, w.H, M, dtype=torch.float32, device="cuda")
    ks = torch.empty(w.batch, w.H, M, 3, w.d, dtype=torch.int16, device="cuda")
    fsl.fs_cell_summaries(k, kbar, a, p, kbar_split=ks)
    sh = fsl.shape_of(k)
    ws = torch.empty(fsl.fs_prune_workspace_bytes(sh, p), dtype=torch.uint8, device="cuda")
    ret = torch.empty(w.batch, w.H, NB, p.P + p.W, dtype=torch.int32, device="cuda")
    nret = torch.empty(w.batch, w.H, NB, dtype=torch.int32, device="cuda")
    fsl.fs_prune_retained(sh, a, ret, nret, ws, p)
    s1 = torch.empty(w.batch, w.H, w.N, p.K, dtype=torch.int32, device="cuda")
    s2 = torch.empty_like(s1)
    print("[gpu] score with and without split operands", flush=True)
    fsl.fs_score_select(q, kbar, a, ret, nret, 4.0, 1.0, s1, p)
    fsl.fs_score_select(q, kbar, a, ret, nret, 4.0, 1.0, s2, p, kbar_split=ks)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("w,p,extra", [
    (synth.Workload(batch=2, H=2, N=2000, d=128, dtype="bf16", seed=72, needle_frac=0.005), fsl.Params(), {}),
    (synth.Workload(batch=1, H=3, N=1500, d=64, dtype="bf16", seed=73, needle_frac=0.01), fsl.Params(P=6, W=2, K=3),
     {"gain": True}),
    (synth.Workload(batch=1, H=2, N=1300, d=128, dtype="bf16", seed=74, needle_frac=0.01), fsl.Params(prune=False),
     {}),
    (synth.Workload(batch=1, H=2, N=1111, d=128, dtype="bf16", seed=75), fsl.Params(P=9, W=3, K=8), {"lam": 0.0}),
    (synth.Workload(batch=1, H=2, N=100, d=64, dtype="bf16", seed=76), fsl.Params(P=2, W=1), {}),
    # content matters: priors close together, so the tile bound holds for some tiles and not others
    (synth.Workload(batch=1, H=4, N=4000, d=128, dtype="bf16", seed=77), fsl.Params(), {"lam": 0.02}),
    (synth.Workload(batch=2, H=2, N=4096, d=128, dtype="bf16", seed=78, needle_frac=0.005), fsl.Params(), {}),
    # content only, and every query feature at index 0 or 1 mod 8 is zero: the tile bound's
    # |q| must come from all features (a norm from one element pair per 16-byte run is
    # 0 here, and then every tile after the first would be passed over)
    (synth.Workload(batch=1, H=2, N=3000, d=128, dtype="bf16", seed=79), fsl.Params(), {"lam": 0.0, "q_gaps": True}),
], ids=["d128", "d64-K3-gain", "FS", "K8-lam0", "one-block", "lam0.02", "needles-4k", "lam0-qgaps"])
def test_fused_route_readout(w, p, extra):
    """fs_select_readout in its single-kernel form gives bitwise the selections and
    outputs of fs_score_select followed by fs_readout, with and without the tile bound
    (kbar_norm) and without the selections output; both meet the oracle."""
    host = pu.inputs(w)
    if extra.get("q_gaps"):
        f = np.arange(w.d) % 8
        host["q"] = host["q"].copy()
        host["q"][..., (f == 0) | (f == 1)] = 0
    q, k, v = (pu.to_device(host[x], w.dtype) for x in "qkv")
    gain_h = synth.gains(97, w.H, w.d) if extra.get("gain") else None
    gain = torch.from_numpy(gain_h).cuda() if gain_h is not None else None
    lam = extra.get("lam", 1.0)
    M, NB = w.N // 32, (w.N + 127) // 128
    kbar = torch.empty(w.batch, w.H, max(M, 1), w.d, dtype=torch.float32, device="cuda")
    a = torch.empty(w.batch, w.H, max(M, 1), dtype=torch.float32, device="cuda")
    ks = torch.empty(w.batch, w.H, max(M, 1), 3, w.d, dtype=torch.int16, device="cuda")
    kn = torch.empty(w.batch, w.H, max(M, 1), dtype=torch.float32, device="cuda")
    fsl.fs_cell_summaries(k, kbar, a, p, kbar_split=ks, kbar_norm=kn)
    ret = nret = None
    if p.prune:
        sh = fsl.shape_of(k)
        ws = torch.empty(fsl.fs_prune_workspace_bytes(sh, p), dtype=torch.uint8, device="cuda")
        ret = torch.empty(w.batch, w.H, NB, p.P + p.W, dtype=torch.int32, device="cuda")
        nret = torch.empty(w.batch, w.H, NB, dtype=torch.int32, device="cuda")
        fsl.fs_prune_retained(sh, a, ret, nret, ws, p)
    s1 = torch.empty(w.batch, w.H, w.N, p.K, dtype=torch.int32, device="cuda")
    s2 = torch.full_like(s1, -7)
    s4 = torch.full_like(s1, -7)
    o1, o2, o3, o4 = (torch.empty_like(q) for _ in range(4))
    print(f"[gpu] fused vs two kernels {w} {p}", flush=True)
    fsl.fs_score_select(q, kbar, a, ret, nret, 4.0, lam, s1, p, kbar_split=ks)
    fsl.fs_readout(q, k, v, s1, gain, o1, p)
    fsl.fs_select_readout(q, k, v, kbar, a, ret, nret, 4.0, lam, gain, o2, s2, p, kbar_split=ks)
    fsl.fs_select_readout(q, k, v, kbar, a, ret, nret, 4.0, lam, gain, o3, None, p, kbar_split=ks)
    fsl.fs_select_readout(q, k, v, kbar, a, ret, nret, 4.0, lam, gain, o4, s4, p, kbar_split=ks, kbar_norm=kn)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(s2, s4)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), o4.view(torch.int16))
    heads = [(b, h) for b in range(w.batch) for h in range(w.H)]
    refs = pu.run_oracle(w, host, p, heads, 4.0, lam, gain_h)
    for name, sel_t, out_t in (("two kernels", s1, o1), ("fused", s2, o2)):
        sel_h, out_h = sel_t.cpu().numpy(), out_t.float().cpu().numpy()
        for (b, h), ref in refs.items():
            pu.compare_head(sel_h[b, h], out_h[b, h], ref, p, w.dtype, what=f"{name} b{b} h{h}")
