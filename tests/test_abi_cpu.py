"""CPU checks of the C ABI: the library loads, exports what include/fsl.h declares,
and rejects bad arguments on the host before anything reaches the GPU (these calls
never touch the HIP runtime, so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import cell_routed_long_amd as fsl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsl.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fsl.LIB_PATH):
        fsl.build()
    return fsl.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fs_\w+)\s*\(", text, flags=re.M)))


def test_exports_match_header(L):
    declared = declared_functions()
    assert {"fs_cell_summaries", "fs_prune_retained", "fs_longrange_prefill", "fs_longrange_decode"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", fsl.LIB_PATH], capture_output=True, text=True, check=True)
    exported = sorted(set(m for m in re.findall(r" T (\w+)", out.stdout)))
    assert exported == declared
    for name in declared:
        assert hasattr(L, name)


def test_status_strings(L):
    for code in range(6):
        assert fsl.status_string(code)


def shape(b=1, H=2, N=1024, d=64, dtype=fsl.FS_F32):
    return fsl.fs_shape(b, H, N, d, dtype)


def prm(**kw):
    return fsl.Params(**kw).c()


def call_summaries(L, sh, p, k=1, kbar=1, a=1):
    vp = ctypes.c_void_p
    return L.fs_cell_summaries(ctypes.byref(sh), ctypes.byref(p), vp(k) if k else None,
                               vp(kbar) if kbar else None, vp(a) if a else None, None, None, None)


@pytest.mark.parametrize("sh,p,expect", [
    (shape(b=0), prm(), fsl.FS_ERR_INVALID),
    (shape(H=0), prm(), fsl.FS_ERR_INVALID),
    (shape(N=0), prm(), fsl.FS_ERR_INVALID),
    (shape(dtype=7), prm(), fsl.FS_ERR_INVALID),
    (shape(), prm(K=0), fsl.FS_ERR_INVALID),
    (shape(), prm(P=-1), fsl.FS_ERR_INVALID),
    (shape(), prm(B=100), fsl.FS_ERR_INVALID),      # B % s != 0
    (shape(), prm(eps=-1.0), fsl.FS_ERR_INVALID),
    (shape(d=96), prm(), fsl.FS_ERR_UNSUPPORTED),
    (shape(H=129), prm(), fsl.FS_ERR_UNSUPPORTED),
    (shape(), prm(K=9), fsl.FS_ERR_UNSUPPORTED),
    (shape(), prm(s=16, B=128), fsl.FS_ERR_UNSUPPORTED),
    (shape(), prm(B=256), fsl.FS_ERR_UNSUPPORTED),
    (shape(), prm(P=1000, W=100), fsl.FS_ERR_UNSUPPORTED),
    (shape(N=(1 << 22) + 1), prm(), fsl.FS_ERR_UNSUPPORTED),
    (shape(b=8, H=128, N=1 << 22), prm(), fsl.FS_ERR_UNSUPPORTED),  # more than 2^26 cells
    (shape(b=512, H=128), prm(), fsl.FS_ERR_UNSUPPORTED),          # batch * H > 65535
])
def test_summaries_rejects_bad_arguments(L, sh, p, expect):
    assert call_summaries(L, sh, p) == expect


def test_null_pointers_rejected(L):
    assert call_summaries(L, shape(), prm(), k=0) == fsl.FS_ERR_INVALID
    assert call_summaries(L, shape(), prm(), a=0) == fsl.FS_ERR_INVALID
    assert L.fs_cell_summaries(None, ctypes.byref(prm()), None, None, None, None, None, None) == fsl.FS_ERR_INVALID


def test_workspace_sizes(L):
    sh, p = shape(b=4, H=16, N=16384, d=128, dtype=fsl.FS_BF16), prm()
    ws = fsl.fs_prefill_workspace_bytes(sh, fsl.Params())
    M, NB = 16384 // 32, 16384 // 128
    # summaries (fp32, bf16 parts and their norms) + key norms + per-cell exit blocks + the cells of every head in
    # priority order (8 bytes each) + retained lists + counts + selections
    at_least = 64 * (M * 128 * 4 + M * 3 * 128 * 2 + M * 4 + M * 4 + M * 4 + M * 8 + NB * 72 * 4 + NB * 4
                     + 16384 * 4 * 4)
    assert at_least <= ws <= at_least + 9 * 256
    assert fsl.fs_prefill_workspace_bytes(shape(d=96), fsl.Params()) == 0
    assert fsl.fs_prune_workspace_bytes(sh, fsl.Params()) >= 64 * M * (4 + 8)


def test_prefill_validation_before_launch(L):
    sh, p = shape(), prm()
    vp = ctypes.c_void_p
    H = sh.H
    ones = (ctypes.c_float * H)(*([4.0] * H))
    lam = (ctypes.c_float * H)(*([1.0] * H))
    bad_sigma = (ctypes.c_float * H)(*([0.0] * H))
    ws = fsl.fs_prefill_workspace_bytes(sh, fsl.Params())
    args = lambda sig, ws_bytes, out=1, q=1: (ctypes.byref(sh), ctypes.byref(p), vp(q) if q else None, vp(1), vp(1),
                                              sig, lam, None, vp(out) if out else None, None, None, 0, vp(1), ws_bytes,
                                              None)
    assert L.fs_longrange_prefill(*args(bad_sigma, ws)) == fsl.FS_ERR_INVALID
    assert L.fs_longrange_prefill(*args(ones, ws - 1)) == fsl.FS_ERR_WORKSPACE
    assert L.fs_longrange_prefill(*args(ones, ws, out=0)) == fsl.FS_ERR_INVALID  # nothing requested
    assert L.fs_longrange_prefill(*args(ones, ws, q=0)) == fsl.FS_ERR_INVALID    # output needs q


def test_prune_requires_fsl_mode(L):
    sh = shape()
    p = prm(prune=False)
    vp = ctypes.c_void_p
    assert L.fs_prune_retained(ctypes.byref(sh), ctypes.byref(p), vp(1), vp(1), vp(1), vp(1), 1 << 20,
                               None) == fsl.FS_ERR_INVALID
    p = prm()
    assert L.fs_prune_retained(ctypes.byref(sh), ctypes.byref(p), vp(1), vp(1), vp(1), vp(1), 0,
                               None) == fsl.FS_ERR_WORKSPACE


# ------------------------------------------------------------------ decode ----

def test_decode_state_bytes(L):
    p = fsl.Params()
    b, H, d = 32, 8, 128
    n = fsl.fs_decode_state_bytes(b, H, d, fsl.FS_BF16, p)
    S = p.P + p.W + p.B // p.s  # retained + pending slots
    per_rec = S * p.s * d * 2 * 2 + S * d * 4  # raw K/V + mean keys
    assert 256 + b * H * per_rec <= n <= 256 + b * H * (per_rec + 8 * 1024)
    assert fsl.fs_decode_state_bytes(b, H, d, fsl.FS_F32, p) > n
    # FS (no pruning) has no bounded state; P + W + B/s above 128 slots is not supported
    assert fsl.fs_decode_state_bytes(b, H, d, fsl.FS_BF16, fsl.Params(prune=False)) == 0
    assert fsl.fs_decode_state_bytes(b, H, d, fsl.FS_BF16, fsl.Params(P=120, W=5)) == 0
    assert fsl.fs_decode_state_bytes(b, H, d, fsl.FS_BF16, fsl.Params(P=120, W=4)) > 0
    assert fsl.fs_decode_state_bytes(0, H, d, fsl.FS_BF16, p) == 0
    assert fsl.fs_decode_state_bytes(b, H, 96, fsl.FS_BF16, p) == 0


def test_decode_validation_before_launch(L):
    p = fsl.Params()
    prm_c = p.c()
    b, H, d = 2, 3, 64
    n = fsl.fs_decode_state_bytes(b, H, d, fsl.FS_F32, p)
    vp = ctypes.c_void_p
    sig = (ctypes.c_float * H)(*([4.0] * H))
    lam = (ctypes.c_float * H)(*([1.0] * H))
    bad = (ctypes.c_float * H)(*([-1.0] * H))

    def call(prm=prm_c, st_bytes=n, sigma=sig, q=1, out=1, state=1, dd=d, dtype=fsl.FS_F32):
        return L.fs_longrange_decode(ctypes.byref(prm), b, H, dd, dtype, vp(state) if state else None, st_bytes,
                                     vp(q) if q else None, vp(1), vp(1), sigma, lam, None,
                                     vp(out) if out else None, None, None)

    assert call(st_bytes=n - 1) == fsl.FS_ERR_STATE
    assert call(st_bytes=n + 256) == fsl.FS_ERR_STATE
    assert call(q=0) == fsl.FS_ERR_INVALID
    assert call(out=0) == fsl.FS_ERR_INVALID
    assert call(state=0) == fsl.FS_ERR_INVALID
    assert call(sigma=bad) == fsl.FS_ERR_INVALID
    assert call(dd=96) == fsl.FS_ERR_UNSUPPORTED
    assert call(dtype=5) == fsl.FS_ERR_INVALID
    assert call(prm=fsl.Params(prune=False).c()) == fsl.FS_ERR_UNSUPPORTED
    assert call(prm=fsl.Params(K=0).c()) == fsl.FS_ERR_INVALID


def test_prefill_state_validation(L):
    sh = shape(b=1, H=2, N=1000, d=64)
    p = fsl.Params()
    vp = ctypes.c_void_p
    sig = (ctypes.c_float * 2)(4.0, 4.0)
    lam = (ctypes.c_float * 2)(1.0, 1.0)
    ws = fsl.fs_prefill_workspace_bytes(sh, p)
    n = fsl.fs_decode_state_bytes(1, 2, 64, fsl.FS_F32, p)

    def call(prm, st_bytes, v=1):
        return L.fs_longrange_prefill(ctypes.byref(sh), ctypes.byref(prm), None, vp(1), vp(v) if v else None, sig,
                                      lam, None, None, None, vp(1), st_bytes, vp(1), ws, None)

    assert call(p.c(), n - 1) == fsl.FS_ERR_STATE
    assert call(p.c(), n, v=0) == fsl.FS_ERR_INVALID            # the state keeps raw values
    assert call(fsl.Params(prune=False).c(), n) == fsl.FS_ERR_UNSUPPORTED


# ------------------------------------------------------------ local branch ----

def test_local_state_bytes(L):
    b, H, d, w = 32, 8, 128, 512
    align = lambda x: (x + 255) // 256 * 256
    rec = 256 + align(w * d * 2) + align(w * d * 2)  # position, rings of the last w keys and values
    # header, (cos, sin) table of offsets 0 .. w, records
    assert fsl.fs_local_state_bytes(b, H, d, fsl.FS_BF16, w) == 256 + align((w + 1) * (d // 2) * 8) + b * H * rec
    assert fsl.fs_local_state_bytes(b, H, d, fsl.FS_F32, w) > fsl.fs_local_state_bytes(b, H, d, fsl.FS_BF16, w)
    assert fsl.fs_local_state_bytes(b, H, d, fsl.FS_BF16, 0) > 0
    for bad in [(b, H, d, fsl.FS_BF16, -1), (b, H, d, fsl.FS_BF16, 65536), (b, H, 96, fsl.FS_BF16, w),
                (0, H, d, fsl.FS_BF16, w), (b, 129, d, fsl.FS_BF16, w), (b, H, d, 3, w)]:
        assert fsl.fs_local_state_bytes(*bad) == 0


def test_local_state_build_validation(L):
    b, H, d, w = 1, 2, 64, 16
    n_bytes = fsl.fs_local_state_bytes(b, H, d, fsl.FS_F32, w)
    vp = ctypes.c_void_p

    def call(n, pos, st_bytes=n_bytes, base=10000.0, state=1, k=1):
        return L.fs_local_state_build(b, H, d, fsl.FS_F32, w, base, vp(state) if state else None, st_bytes,
                                      vp(k) if k else None, vp(1), n, pos, None)

    assert call(5, 4) == fsl.FS_ERR_INVALID            # more tokens than positions before pos
    assert call(10, 100) == fsl.FS_ERR_INVALID         # fewer than the w tokens the window needs
    assert call(3, 5) == fsl.FS_ERR_INVALID            # pos < w: all pos tokens are needed
    assert call(-1, 0) == fsl.FS_ERR_INVALID
    assert call(16, 100, base=1.0) == fsl.FS_ERR_INVALID
    assert call(16, 100, state=0) == fsl.FS_ERR_INVALID
    assert call(16, 100, k=0) == fsl.FS_ERR_INVALID
    assert call(16, 100, st_bytes=n_bytes - 1) == fsl.FS_ERR_STATE


def test_local_decode_validation(L):
    b, H, d, w = 1, 2, 64, 16
    n_bytes = fsl.fs_local_state_bytes(b, H, d, fsl.FS_F32, w)
    vp = ctypes.c_void_p
    alpha = (ctypes.c_float * H)(1.0, 1.0)
    nan_alpha = (ctypes.c_float * H)(1.0, float("nan"))

    def call(st_bytes=n_bytes, q=1, out=1, al=None, o_lr=None, ww=w):
        return L.fs_local_decode(b, H, d, fsl.FS_F32, ww, vp(1), st_bytes, vp(q) if q else None, vp(1), vp(1), al,
                                 vp(o_lr) if o_lr else None, vp(out) if out else None, None)

    assert call(q=0) == fsl.FS_ERR_INVALID
    assert call(out=0) == fsl.FS_ERR_INVALID
    assert call(o_lr=1) == fsl.FS_ERR_INVALID           # o_lr without alpha_h
    assert call(o_lr=1, al=nan_alpha) == fsl.FS_ERR_INVALID
    assert call(st_bytes=n_bytes + 256) == fsl.FS_ERR_STATE
    assert call(ww=-1) == fsl.FS_ERR_INVALID
    assert call(ww=w + 1) == fsl.FS_ERR_STATE          # a state for another w has another size


def test_attention_decode_validation(L):
    """fs_attention_decode checks both states' sizes and every argument of the two
    steps it fuses on the host, before any HIP call."""
    p = fsl.Params()
    prm_c = p.c()
    b, H, d, w = 2, 3, 64, 16
    n = fsl.fs_decode_state_bytes(b, H, d, fsl.FS_F32, p)
    nl = fsl.fs_local_state_bytes(b, H, d, fsl.FS_F32, w)
    vp = ctypes.c_void_p
    sig = (ctypes.c_float * H)(*([4.0] * H))
    lam = (ctypes.c_float * H)(*([1.0] * H))
    alpha = (ctypes.c_float * H)(*([0.5] * H))
    nan_alpha = (ctypes.c_float * H)(0.5, float("nan"), 0.5)
    bad_sig = (ctypes.c_float * H)(*([0.0] * H))

    def call(prm=prm_c, st=n, lst=nl, ww=w, q=1, out=1, state=1, lstate=1, al=alpha, sigma=sig, dd=d, bb=b):
        return L.fs_attention_decode(ctypes.byref(prm), bb, H, dd, fsl.FS_F32, vp(state) if state else None, st, ww,
                                     vp(lstate) if lstate else None, lst, vp(q) if q else None, vp(1), vp(1), sigma,
                                     lam, None, al, vp(out) if out else None, None, None)

    assert call(st=n + 256) == fsl.FS_ERR_STATE
    assert call(lst=nl - 1) == fsl.FS_ERR_STATE
    assert call(ww=w + 1) == fsl.FS_ERR_STATE           # the local state of another window has another size
    assert call(state=0) == fsl.FS_ERR_INVALID
    assert call(lstate=0) == fsl.FS_ERR_INVALID
    assert call(q=0) == fsl.FS_ERR_INVALID
    assert call(out=0) == fsl.FS_ERR_INVALID
    assert call(al=None) == fsl.FS_ERR_INVALID          # Eq. 2 needs alpha_h
    assert call(al=nan_alpha) == fsl.FS_ERR_INVALID
    assert call(sigma=bad_sig) == fsl.FS_ERR_INVALID
    assert call(ww=-1) == fsl.FS_ERR_INVALID
    assert call(ww=65536) == fsl.FS_ERR_UNSUPPORTED
    assert call(dd=96) == fsl.FS_ERR_UNSUPPORTED
    assert call(bb=30000) == fsl.FS_ERR_UNSUPPORTED     # batch * H above 65535
    assert call(prm=fsl.Params(prune=False).c()) == fsl.FS_ERR_UNSUPPORTED
    assert call(prm=fsl.Params(K=0).c()) == fsl.FS_ERR_INVALID


def test_local_window_validation(L):
    sh = shape(b=1, H=2, N=256, d=64)
    vp = ctypes.c_void_p
    alpha = (ctypes.c_float * 2)(1.0, 1.0)

    def call(w=512, base=10000.0, q=1, o_lr=None, al=None):
        return L.fs_local_window(ctypes.byref(sh), w, base, vp(q) if q else None, vp(1), vp(1), al,
                                 vp(o_lr) if o_lr else None, vp(1), None)

    assert call(q=0) == fsl.FS_ERR_INVALID
    assert call(w=-1) == fsl.FS_ERR_INVALID
    assert call(base=1.0) == fsl.FS_ERR_INVALID
    assert call(o_lr=1) == fsl.FS_ERR_INVALID            # o_lr without alpha_h
    assert call(w=65536) == fsl.FS_ERR_UNSUPPORTED       # past the largest window
    assert call(w=65536, o_lr=1, al=alpha) == fsl.FS_ERR_UNSUPPORTED


def test_noalloc_prefill_rejects_before_launch(L):
    """fs_longrange_prefill_noalloc checks its arguments and the workspace the shape needs
    against its fixed scratch on the host, before any HIP call."""
    cap = fsl.fs_noalloc_scratch_bytes()
    assert cap == 32 << 20
    vp = ctypes.c_void_p
    H = 16
    sig = (ctypes.c_float * H)(*[4.0] * H)
    lam = (ctypes.c_float * H)(*[1.0] * H)
    p = prm()
    big = shape(b=4, H=H, N=16384, d=128, dtype=fsl.FS_BF16)
    assert fsl.fs_prefill_workspace_bytes(big) > cap
    assert L.fs_longrange_prefill_noalloc(ctypes.byref(big), ctypes.byref(p), vp(1), vp(1), vp(1), sig, lam, None,
                                          vp(1), None, None, 0, None) == fsl.FS_ERR_WORKSPACE
    fits = shape(b=2, H=H, N=16384, d=128, dtype=fsl.FS_BF16)
    assert fsl.fs_prefill_workspace_bytes(fits) <= cap
    # invalid arguments are reported as for fs_longrange_prefill, also where the shape would not fit
    assert L.fs_longrange_prefill_noalloc(ctypes.byref(big), ctypes.byref(p), vp(1), None, vp(1), sig, lam, None,
                                          vp(1), None, None, 0, None) == fsl.FS_ERR_INVALID
    assert L.fs_longrange_prefill_noalloc(ctypes.byref(fits), ctypes.byref(p), vp(1), vp(1), vp(1), sig, lam, None,
                                          None, None, None, 0, None) == fsl.FS_ERR_INVALID


def test_fsb_validation_before_launch(L):
    """fs_fsb_prefill rejects bad arguments on the host (FS-B: Sec. 3.4)."""
    vp = ctypes.c_void_p
    H = 2
    sig = (ctypes.c_float * H)(4.0, 4.0)
    lam = (ctypes.c_float * H)(1.0, 1.0)
    tau = (ctypes.c_float * H)(1.0, 1.0)
    tau_nan = (ctypes.c_float * H)(1.0, float("nan"))
    sh = shape(b=1, H=H, N=4096, d=128, dtype=fsl.FS_BF16)
    p = prm()
    fb = fsl.FsbParams().c_struct()
    need = L.fs_fsb_workspace_bytes(ctypes.byref(sh), ctypes.byref(p), ctypes.byref(fb))
    assert need > 0

    def call(sh=sh, fb=fb, q=1, k=1, v=1, out=1, sel=None, cand=None, t=tau, ws=need):
        return L.fs_fsb_prefill(ctypes.byref(sh), ctypes.byref(p), ctypes.byref(fb), vp(q) if q else None,
                                vp(k) if k else None, vp(v) if v else None, sig, lam, t, None,
                                vp(out) if out else None, vp(sel) if sel else None, vp(cand) if cand else None,
                                vp(1), ws, None)

    assert call(q=0) == fsl.FS_ERR_INVALID
    assert call(k=0) == fsl.FS_ERR_INVALID
    assert call(v=0) == fsl.FS_ERR_INVALID                  # out needs v
    assert call(out=0) == fsl.FS_ERR_INVALID                # nothing to write
    assert call(t=None) == fsl.FS_ERR_INVALID
    assert call(t=tau_nan) == fsl.FS_ERR_INVALID
    assert call(ws=need - 1) == fsl.FS_ERR_WORKSPACE
    assert call(fb=fsl.FsbParams(Wb=0).c_struct()) == fsl.FS_ERR_INVALID
    assert call(fb=fsl.FsbParams(c=-1.0).c_struct()) == fsl.FS_ERR_INVALID
    assert call(fb=fsl.FsbParams(Wb=17).c_struct()) == fsl.FS_ERR_UNSUPPORTED
    big = shape(b=1, H=H, N=131200 + 128, d=128, dtype=fsl.FS_BF16)  # 4100 cells available to the last block
    assert L.fs_fsb_workspace_bytes(ctypes.byref(big), ctypes.byref(p), ctypes.byref(fb)) == 0
    assert call(sh=big) == fsl.FS_ERR_UNSUPPORTED
    edge = shape(b=1, H=H, N=131200, d=128, dtype=fsl.FS_BF16)  # exactly 4096
    assert L.fs_fsb_workspace_bytes(ctypes.byref(edge), ctypes.byref(p), ctypes.byref(fb)) > 0


def test_chunk_and_state_init_validation(L):
    """fs_decode_state_init and fs_longrange_prefill_chunk reject bad arguments on the host."""
    vp = ctypes.c_void_p
    b, H, d = 1, 2, 64
    p = prm()
    n_bytes = fsl.fs_decode_state_bytes(b, H, d, fsl.FS_BF16)
    sig = (ctypes.c_float * H)(4.0, 4.0)
    lam = (ctypes.c_float * H)(1.0, 1.0)
    assert L.fs_decode_state_init(ctypes.byref(p), b, H, d, fsl.FS_BF16, None, n_bytes, None) == fsl.FS_ERR_INVALID
    assert L.fs_decode_state_init(ctypes.byref(p), b, H, d, fsl.FS_BF16, vp(1), n_bytes + 1, None) == fsl.FS_ERR_STATE
    fs_p = prm(prune=False)
    assert L.fs_decode_state_init(ctypes.byref(fs_p), b, H, d, fsl.FS_BF16, vp(1), n_bytes, None) == \
        fsl.FS_ERR_UNSUPPORTED

    def chunk(n=16, st=n_bytes, q=1, out=1):
        return L.fs_longrange_prefill_chunk(ctypes.byref(p), b, H, d, fsl.FS_BF16, vp(1), st, n, vp(q) if q else None,
                                            vp(1), vp(1), sig, lam, None, vp(out) if out else None, None, None)

    assert chunk(n=0) == fsl.FS_ERR_INVALID
    assert chunk(q=0) == fsl.FS_ERR_INVALID
    assert chunk(out=0) == fsl.FS_ERR_INVALID
    assert chunk(st=n_bytes - 256) == fsl.FS_ERR_STATE
    assert chunk(n=65537) == fsl.FS_ERR_UNSUPPORTED


def test_readout_backward_validation_before_launch(L):
    """fs_readout_backward rejects bad arguments on the host (readout backward: Sec. 3.3
    "Training"), and its workspace covers du, lse, Delta, the cell masks and the gain partials."""
    vp = ctypes.c_void_p
    b, H, N, d = 2, 3, 4096, 64
    sh = shape(b=b, H=H, N=N, d=d, dtype=fsl.FS_BF16)
    p = prm()
    need = L.fs_readout_backward_workspace_bytes(ctypes.byref(sh), ctypes.byref(p))
    M, NB, K = N // 32, N // 128, 4
    extra = -(-N * K // 512)  # chunks of 512 queries beyond one per cell
    core = b * H * (N * d * 4 + 2 * N * 4 + M * NB * 16 + NB * d * 4)
    tables = b * H * (2 * (M + 1) * 4 + (M + extra) * 4 + (extra + 1) * 4 + 2 * extra * 2 * 32 * d * 4) \
        + H * 32 * d * 4
    assert core + tables <= need < core + tables + 11 * 256

    def call(sh=sh, q=1, k=1, v=1, sel=1, dout=1, dq=1, dk=1, dv=1, ws=need, wsp=1):
        f = lambda x: vp(x) if x else None
        return L.fs_readout_backward(ctypes.byref(sh), ctypes.byref(p), f(q), f(k), f(v), f(sel), None, f(dout),
                                     f(dq), f(dk), f(dv), None, f(wsp), ws, None)

    for name in ("q", "k", "v", "sel", "dout", "dq", "dk", "dv", "wsp"):
        assert call(**{name: 0}) == fsl.FS_ERR_INVALID, name
    assert call(ws=need - 1) == fsl.FS_ERR_WORKSPACE
    big = shape(b=1, H=1, N=65536 + 1, d=d, dtype=fsl.FS_BF16)
    assert L.fs_readout_backward_workspace_bytes(ctypes.byref(big), ctypes.byref(p)) == 0
    assert call(sh=big) == fsl.FS_ERR_UNSUPPORTED
    edge = shape(b=1, H=1, N=65536, d=d, dtype=fsl.FS_BF16)
    assert L.fs_readout_backward_workspace_bytes(ctypes.byref(edge), ctypes.byref(p)) > 0
    wide = shape(b=4096, H=128, N=1024, d=d, dtype=fsl.FS_BF16)  # 2^24 cells: the key side's grid is too large
    assert call(sh=wide) == fsl.FS_ERR_UNSUPPORTED
    assert call(sh=shape(b=1, H=1, N=4096, d=96, dtype=fsl.FS_BF16)) == fsl.FS_ERR_UNSUPPORTED
    assert L.fs_readout_backward_workspace_bytes(ctypes.byref(sh), ctypes.byref(prm(K=9))) == 0
