"""Python binding of libfsl.so, the gfx950 implementation of FreeSolo's
long-range sparse-attention branch (FS / FS-L).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fsl.h.  PyTorch supplies device
memory and the current stream.  If the library has not been built, every call
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from ._build import LIB_PATH, build  # noqa: F401

FS_OK, FS_ERR_INVALID, FS_ERR_UNSUPPORTED, FS_ERR_WORKSPACE, FS_ERR_STATE, FS_ERR_HIP = range(6)
FS_F32, FS_BF16 = 0, 1
FS_MAX_HEADS = 128


class FslError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class fs_params(ctypes.Structure):
    _fields_ = [("s", ctypes.c_int32), ("B", ctypes.c_int32), ("P", ctypes.c_int32), ("W", ctypes.c_int32),
                ("K", ctypes.c_int32), ("prune", ctypes.c_int32), ("eps", ctypes.c_float)]


class fs_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int64), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class fs_fsb_params(ctypes.Structure):
    _fields_ = [("Wb", ctypes.c_int32), ("c", ctypes.c_float)]


@dataclass(frozen=True)
class FsbParams:
    """FS-B search parameters (Sec. 3.4): beam width W^b and the radius weight c of Eq. 11."""
    Wb: int = 16
    c: float = 8.0

    def c_struct(self) -> fs_fsb_params:
        return fs_fsb_params(self.Wb, self.c)


@dataclass(frozen=True)
class Params:
    """Method parameters; defaults are the page's (App. A)."""
    s: int = 32
    B: int = 128
    P: int = 64
    W: int = 8
    K: int = 4
    prune: bool = True
    eps: float = 1e-8

    def c(self) -> fs_params:
        return fs_params(self.s, self.B, self.P, self.W, self.K, int(self.prune), self.eps)


_lib = None


def lib():
    """The loaded libfsl.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        # FSL_LIBRARY: an instrumented build of the same sources (the sanitizer test)
        path = os.environ.get("FSL_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with cell_routed_long_amd.build()")
        L = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        P_shape, P_prm = ctypes.POINTER(fs_shape), ctypes.POINTER(fs_params)
        L.fs_status_string.argtypes = [ctypes.c_int]
        L.fs_status_string.restype = ctypes.c_char_p
        L.fs_cell_summaries.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp]
        L.fs_prune_workspace_bytes.argtypes = [P_shape, P_prm]
        L.fs_prune_workspace_bytes.restype = sz
        L.fs_prune_retained.argtypes = [P_shape, P_prm, vp, vp, vp, vp, sz, vp]
        L.fs_score_select.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.fs_readout.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp]
        L.fs_select_readout.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.fs_readout_backward_workspace_bytes.argtypes = [P_shape, P_prm]
        L.fs_readout_backward_workspace_bytes.restype = sz
        L.fs_readout_backward.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fs_prefill_workspace_bytes.argtypes = [P_shape, P_prm]
        L.fs_prefill_workspace_bytes.restype = sz
        L.fs_longrange_prefill.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
        L.fs_noalloc_scratch_bytes.argtypes = []
        L.fs_noalloc_scratch_bytes.restype = sz
        L.fs_longrange_prefill_noalloc.argtypes = [P_shape, P_prm, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        P_fsb = ctypes.POINTER(fs_fsb_params)
        L.fs_fsb_workspace_bytes.argtypes = [P_shape, P_prm, P_fsb]
        L.fs_fsb_workspace_bytes.restype = sz
        L.fs_fsb_prefill.argtypes = [P_shape, P_prm, P_fsb, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        i32_, i64_ = ctypes.c_int32, ctypes.c_int64
        L.fs_decode_state_init.argtypes = [P_prm, i32_, i32_, i32_, ctypes.c_int, vp, sz, vp]
        L.fs_longrange_prefill_chunk.argtypes = [P_prm, i32_, i32_, i32_, ctypes.c_int, vp, sz, i64_, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, vp]
        L.fs_decode_state_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, P_prm]
        L.fs_decode_state_bytes.restype = sz
        L.fs_longrange_decode.argtypes = [P_prm, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                          vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.fs_local_window.argtypes = [P_shape, ctypes.c_int64, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp]
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.fs_local_state_bytes.argtypes = [i32, i32, i32, ctypes.c_int, i64]
        L.fs_local_state_bytes.restype = sz
        L.fs_local_state_build.argtypes = [i32, i32, i32, ctypes.c_int, i64, ctypes.c_float, vp, sz, vp, vp, i64,
                                           i64, vp]
        L.fs_local_decode.argtypes = [i32, i32, i32, ctypes.c_int, i64, vp, sz, vp, vp, vp, vp, vp, vp, vp]
        L.fs_attention_decode.argtypes = [P_prm, i32, i32, i32, ctypes.c_int, vp, sz, i64, vp, sz, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp]
        for name in ("fs_cell_summaries", "fs_prune_retained", "fs_score_select", "fs_readout", "fs_readout_backward",
                     "fs_select_readout", "fs_longrange_prefill", "fs_longrange_prefill_noalloc", "fs_fsb_prefill",
                     "fs_longrange_decode", "fs_decode_state_init", "fs_longrange_prefill_chunk",
                     "fs_local_window",
                     "fs_local_state_build", "fs_local_decode", "fs_attention_decode"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fs_status_string(status).decode()


def _check(status: int, where: str):
    if status != FS_OK:
        raise FslError(status, where)


# ---------------------------------------------------------------- marshalling --

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FS_F32
    if t.dtype == torch.bfloat16:
        return FS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def shape_of(x) -> fs_shape:
    """fs_shape of a [batch, H, N, d] tensor."""
    b, H, N, d = x.shape
    return fs_shape(b, H, N, d, _dtype_code(x))


def _floats(vals, H):
    if isinstance(vals, (int, float)):
        vals = [float(vals)] * H
    arr = (ctypes.c_float * H)(*[float(x) for x in vals])
    return arr


# ------------------------------------------------------------- C ABI calls --

def fs_cell_summaries(k, kbar, a, params: Params = Params(), stream=None, kbar_split=None, kbar_norm=None):
    """Eq. 5: kbar [b,H,N/s,d] fp32 and a [b,H,N/s] fp32 from k [b,H,N,d]; optionally
    kbar_split [b,H,N/s,3,d] (int16/bf16 storage): the bf16 hi/mid/lo parts of kbar, and
    kbar_norm [b,H,N/s] fp32: the norms of kbar."""
    sh, prm = shape_of(k), params.c()
    _check(lib().fs_cell_summaries(ctypes.byref(sh), ctypes.byref(prm), _ptr(k), _ptr(kbar), _ptr(a),
                                   _ptr(kbar_split), _ptr(kbar_norm), _stream(stream)), "fs_cell_summaries")


def fs_prune_workspace_bytes(sh: fs_shape, params: Params = Params()) -> int:
    prm = params.c()
    return int(lib().fs_prune_workspace_bytes(ctypes.byref(sh), ctypes.byref(prm)))


def fs_prune_retained(sh: fs_shape, a, retained, n_retained, workspace, params: Params = Params(), stream=None):
    """Eqs. 6 and 8: retained [b,H,NB,P+W] int32 and n_retained [b,H,NB] int32 from a."""
    prm = params.c()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fs_prune_retained(ctypes.byref(sh), ctypes.byref(prm), _ptr(a), _ptr(retained), _ptr(n_retained),
                                   _ptr(workspace), nbytes, _stream(stream)), "fs_prune_retained")


def fs_score_select(q, kbar, a, retained, n_retained, sigma_h, lambda_h, sel, params: Params = Params(),
                    stream=None, kbar_split=None):
    """Eq. 7 scores and per-query top-K: sel [b,H,N,K] int32 (kbar_split: see fs_cell_summaries)."""
    sh, prm = shape_of(q), params.c()
    sig, lam = _floats(sigma_h, sh.H), _floats(lambda_h, sh.H)
    _check(lib().fs_score_select(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(kbar), _ptr(kbar_split), _ptr(a),
                                 _ptr(retained), _ptr(n_retained), sig, lam, _ptr(sel), _stream(stream)),
           "fs_score_select")


def fs_readout(q, k, v, sel, gain, out, params: Params = Params(), stream=None):
    """Eq. 9 readout with Eq. 17 RMSNorm: out [b,H,N,d]."""
    sh, prm = shape_of(q), params.c()
    _check(lib().fs_readout(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(gain),
                            _ptr(out), _stream(stream)), "fs_readout")


def fs_readout_backward_workspace_bytes(sh: fs_shape, params: Params = Params()) -> int:
    prm = params.c()
    return int(lib().fs_readout_backward_workspace_bytes(ctypes.byref(sh), ctypes.byref(prm)))


def fs_readout_backward(q, k, v, sel, gain, dout, dq, dk, dv, dgain, workspace, params: Params = Params(),
                        stream=None):
    """Backward of fs_readout through the fixed selection sel: dq, dk, dv [b,H,N,d] fp32 and
    dgain [H,d] fp32 (when gain is given); see include/fsl.h."""
    sh, prm = shape_of(q), params.c()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().fs_readout_backward(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
                                     _ptr(gain), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgain),
                                     _ptr(workspace), ws_bytes, _stream(stream)), "fs_readout_backward")


def readout_backward(q, k, v, sel, dout, gain=None, params: Params = Params(), workspace=None, stream=None):
    """Allocate the gradients and workspace with torch and run fs_readout_backward.
    Returns (dq, dk, dv, dgain or None, workspace)."""
    import torch
    sh = shape_of(q)
    ws_bytes = fs_readout_backward_workspace_bytes(sh, params)
    if ws_bytes == 0:
        raise FslError(FS_ERR_UNSUPPORTED, "fs_readout_backward_workspace_bytes")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dgain = torch.empty(sh.H, sh.d, dtype=torch.float32, device=q.device) if gain is not None else None
    fs_readout_backward(q, k, v, sel, gain, dout, dq, dk, dv, dgain, workspace, params, stream)
    return dq, dk, dv, dgain, workspace


def fs_select_readout(q, k, v, kbar, a, retained, n_retained, sigma_h, lambda_h, gain, out, sel=None,
                      params: Params = Params(), stream=None, kbar_split=None, kbar_norm=None):
    """fs_score_select + fs_readout in one call (one kernel for bf16 with kbar_split; with
    kbar_norm too, tiles of cells that no query can select are passed over)."""
    sh, prm = shape_of(q), params.c()
    sig, lam = _floats(sigma_h, sh.H), _floats(lambda_h, sh.H)
    _check(lib().fs_select_readout(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), _ptr(kbar),
                                   _ptr(kbar_split), _ptr(kbar_norm), _ptr(a), _ptr(retained), _ptr(n_retained),
                                   sig, lam,
                                   _ptr(gain), _ptr(out), _ptr(sel), _stream(stream)), "fs_select_readout")


def fs_prefill_workspace_bytes(sh: fs_shape, params: Params = Params()) -> int:
    prm = params.c()
    return int(lib().fs_prefill_workspace_bytes(ctypes.byref(sh), ctypes.byref(prm)))


def fs_longrange_prefill(q, k, v, sigma_h, lambda_h, gain, out, sel, state, workspace,
                         params: Params = Params(), stream=None):
    """The branch over a whole prompt (Eqs. 5-9, 17); see include/fsl.h."""
    sh, prm = shape_of(k), params.c()
    H = sh.H
    sig, lam = _floats(sigma_h, H), _floats(lambda_h, H)
    st_bytes = 0 if state is None else state.numel() * state.element_size()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().fs_longrange_prefill(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), sig, lam,
                                      _ptr(gain), _ptr(out), _ptr(sel), _ptr(state), st_bytes, _ptr(workspace),
                                      ws_bytes, _stream(stream)), "fs_longrange_prefill")


def fs_noalloc_scratch_bytes() -> int:
    return int(lib().fs_noalloc_scratch_bytes())


def fs_longrange_prefill_noalloc(q, k, v, sigma_h, lambda_h, gain, out, sel, state=None,
                                 params: Params = Params(), stream=None):
    """fs_longrange_prefill with the library's fixed device scratch as workspace (no
    allocation anywhere); see include/fsl.h."""
    sh, prm = shape_of(k), params.c()
    H = sh.H
    sig, lam = _floats(sigma_h, H), _floats(lambda_h, H)
    st_bytes = 0 if state is None else state.numel() * state.element_size()
    _check(lib().fs_longrange_prefill_noalloc(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), sig,
                                              lam, _ptr(gain), _ptr(out), _ptr(sel), _ptr(state), st_bytes,
                                              _stream(stream)), "fs_longrange_prefill_noalloc")


def fs_decode_state_bytes(batch: int, H: int, d: int, dtype_code: int, params: Params = Params()) -> int:
    prm = params.c()
    return int(lib().fs_decode_state_bytes(batch, H, d, dtype_code, ctypes.byref(prm)))


def fs_longrange_decode(state, q, k_new, v_new, sigma_h, lambda_h, gain, out, sel=None,
                        params: Params = Params(), stream=None):
    """One decode step for every sequence; q, k_new, v_new, out are [b, H, d]."""
    prm = params.c()
    b, H, d = q.shape
    sig, lam = _floats(sigma_h, H), _floats(lambda_h, H)
    _check(lib().fs_longrange_decode(ctypes.byref(prm), b, H, d, _dtype_code(q), _ptr(state),
                                     state.numel() * state.element_size(), _ptr(q), _ptr(k_new), _ptr(v_new), sig,
                                     lam, _ptr(gain), _ptr(out), _ptr(sel), _stream(stream)), "fs_longrange_decode")


def fs_fsb_workspace_bytes(sh: fs_shape, params: Params = Params(), fsb: FsbParams = FsbParams()) -> int:
    prm, fb = params.c(), fsb.c_struct()
    return int(lib().fs_fsb_workspace_bytes(ctypes.byref(sh), ctypes.byref(prm), ctypes.byref(fb)))


def fs_fsb_prefill(q, k, v, sigma_h, lambda_h, tau_h, gain, out, sel, cand, workspace, params: Params = Params(),
                   fsb: FsbParams = FsbParams(), stream=None):
    """FS-B over a whole prompt (Sec. 3.4; App. E.1); see include/fsl.h."""
    sh, prm, fb = shape_of(k), params.c(), fsb.c_struct()
    H = sh.H
    sig, lam, tau = _floats(sigma_h, H), _floats(lambda_h, H), _floats(tau_h, H)
    _check(lib().fs_fsb_prefill(ctypes.byref(sh), ctypes.byref(prm), ctypes.byref(fb), _ptr(q), _ptr(k), _ptr(v), sig,
                                lam, tau, _ptr(gain), _ptr(out), _ptr(sel), _ptr(cand), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)), "fs_fsb_prefill")


def fs_decode_state_init(state, batch: int, H: int, d: int, dtype, params: Params = Params(), stream=None):
    """An empty decode state at position 0 (dtype: a torch dtype)."""
    import torch
    code = FS_BF16 if dtype == torch.bfloat16 else FS_F32
    prm = params.c()
    _check(lib().fs_decode_state_init(ctypes.byref(prm), batch, H, d, code, _ptr(state),
                                      state.numel() * state.element_size(), _stream(stream)), "fs_decode_state_init")


def fs_longrange_prefill_chunk(state, q, k, v, sigma_h, lambda_h, gain, out, sel=None, params: Params = Params(),
                               stream=None):
    """Chunked prefill into a decode state: q, k, v, out [b, H, n, d], sel [b, H, n, K] or None."""
    prm = params.c()
    b, H, n, d = q.shape
    sig, lam = _floats(sigma_h, H), _floats(lambda_h, H)
    _check(lib().fs_longrange_prefill_chunk(ctypes.byref(prm), b, H, d, _dtype_code(q), _ptr(state),
                                            state.numel() * state.element_size(), n, _ptr(q), _ptr(k), _ptr(v), sig,
                                            lam, _ptr(gain), _ptr(out), _ptr(sel), _stream(stream)),
           "fs_longrange_prefill_chunk")


def prefill_chunk(state, q, k, v, params: Params = Params(), sigma=4.0, lam=1.0, gain=None, want_sel=True,
                  out=None, sel=None, stream=None):
    """Allocate the outputs with torch and run fs_longrange_prefill_chunk; returns (out, sel or None)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if want_sel and sel is None:
        sel = torch.empty(*q.shape[:3], params.K, dtype=torch.int32, device=q.device)
    fs_longrange_prefill_chunk(state, q, k, v, sigma, lam, gain, out, sel if want_sel else None, params, stream)
    return out, (sel if want_sel else None)


# ------------------------------------------------------- allocation helpers --

def new_state(batch: int, H: int, d: int, dtype, params: Params = Params(), device="cuda"):
    """A decode-state buffer (uint8 tensor) of fs_decode_state_bytes for this shape."""
    import torch
    code = FS_BF16 if dtype == torch.bfloat16 else FS_F32
    n = fs_decode_state_bytes(batch, H, d, code, params)
    if n == 0:
        raise FslError(FS_ERR_UNSUPPORTED, "fs_decode_state_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(q, k, v, params: Params = Params(), sigma=4.0, lam=1.0, gain=None, want_out=True, want_sel=True,
            workspace=None, stream=None, state=None):
    """Allocate outputs and workspace with torch and run fs_longrange_prefill.

    `state`, if given (see new_state), is filled for continuing at position N.
    Returns (out or None, sel or None, workspace)."""
    import torch
    sh = shape_of(k)
    ws_bytes = fs_prefill_workspace_bytes(sh, params)
    if ws_bytes == 0:
        raise FslError(FS_ERR_UNSUPPORTED, "fs_prefill_workspace_bytes")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    out = torch.empty_like(k) if want_out else None
    sel = torch.empty(k.shape[0], k.shape[1], k.shape[2], params.K, dtype=torch.int32, device=k.device) \
        if want_sel else None
    fs_longrange_prefill(q, k, v, sigma, lam, gain, out, sel, state, workspace, params, stream)
    return out, sel, workspace


def decode(state, q, k_new, v_new, params: Params = Params(), sigma=4.0, lam=1.0, gain=None, want_sel=True,
           out=None, sel=None, stream=None):
    """One decode step (fs_longrange_decode) for [batch, H, d] inputs; returns (out, sel or None)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if want_sel and sel is None:
        sel = torch.empty(q.shape[0], q.shape[1], params.K, dtype=torch.int32, device=q.device)
    fs_longrange_decode(state, q, k_new, v_new, sigma, lam, gain, out, sel if want_sel else None, params, stream)
    return out, (sel if want_sel else None)


def fs_local_window(q, k, v, out, w: int = 512, rope_base: float = 10000.0, alpha=None, o_lr=None, stream=None):
    """Local branch (Sec. 3.2, Eqs. 3-4) into out [b,H,N,d]; with o_lr and alpha [H],
    out = o_sr + alpha_h * o_lr (Eq. 2).  out may be o_lr."""
    sh = shape_of(q)
    al = None if alpha is None else _floats(alpha, sh.H)
    _check(lib().fs_local_window(ctypes.byref(sh), int(w), float(rope_base), _ptr(q), _ptr(k), _ptr(v), al,
                                 _ptr(o_lr), _ptr(out), _stream(stream)), "fs_local_window")


def local(q, k, v, w: int = 512, rope_base: float = 10000.0, alpha=None, o_lr=None):
    """Allocate the output with torch and run fs_local_window; returns it."""
    import torch
    out = torch.empty_like(q)
    fs_local_window(q, k, v, out, w, rope_base, alpha, o_lr)
    return out



def fs_local_state_bytes(batch: int, H: int, d: int, dtype_code: int, w: int = 512) -> int:
    return int(lib().fs_local_state_bytes(batch, H, d, dtype_code, int(w)))


def fs_local_state_build(state, k, v, pos: int, w: int = 512, rope_base: float = 10000.0, stream=None):
    """Fill a local decode state (uint8 tensor of fs_local_state_bytes) from k, v [b,H,n,d]:
    the raw keys and values at positions pos - n .. pos - 1 (n = 0 for an empty prefix)."""
    b, Hh, n, d = k.shape
    code = _dtype_code(k)
    _check(lib().fs_local_state_build(b, Hh, d, code, int(w), float(rope_base), _ptr(state),
                                      state.numel() * state.element_size(), _ptr(k), _ptr(v), n, int(pos),
                                      _stream(stream)), "fs_local_state_build")


def fs_local_decode(state, q, k_new, v_new, out, w: int = 512, alpha=None, o_lr=None, stream=None):
    """One local-branch decode step for [batch, H, d] inputs into out; with o_lr and
    alpha [H], out = o_sr + alpha_h * o_lr (Eq. 2).  out may be o_lr."""
    b, H, d = q.shape
    al = None if alpha is None else _floats(alpha, H)
    _check(lib().fs_local_decode(b, H, d, _dtype_code(q), int(w), _ptr(state), state.numel() * state.element_size(),
                                 _ptr(q), _ptr(k_new), _ptr(v_new), al, _ptr(o_lr), _ptr(out), _stream(stream)),
           "fs_local_decode")


def fs_attention_decode(state, local_state, q, k_new, v_new, out, alpha, sel=None, params: Params = Params(),
                        sigma=4.0, lam=1.0, gain=None, w: int = 512, stream=None):
    """The whole attention decode step in one launch: out = o_sr + alpha_h * o_lr (Eq. 2)
    from the long-range state and the local state (window w) for [batch, H, d] inputs."""
    prm = params.c()
    b, H, d = q.shape
    sig, la, al = _floats(sigma, H), _floats(lam, H), _floats(alpha, H)
    _check(lib().fs_attention_decode(ctypes.byref(prm), b, H, d, _dtype_code(q), _ptr(state),
                                     state.numel() * state.element_size(), int(w), _ptr(local_state),
                                     local_state.numel() * local_state.element_size(), _ptr(q), _ptr(k_new),
                                     _ptr(v_new), sig, la, _ptr(gain), al, _ptr(out), _ptr(sel), _stream(stream)),
           "fs_attention_decode")


def new_local_state(batch: int, H: int, d: int, dtype, w: int = 512, device="cuda"):
    """A local decode-state buffer (uint8 tensor of fs_local_state_bytes)."""
    import torch
    code = FS_BF16 if dtype == torch.bfloat16 else FS_F32
    n = fs_local_state_bytes(batch, H, d, code, w)
    if n == 0:
        raise FslError(FS_ERR_UNSUPPORTED, "fs_local_state_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def fsb_prefill(q, k, v, tau, params: Params = Params(), fsb: FsbParams = FsbParams(), sigma=4.0, lam=1.0,
                gain=None, want_out=True, want_sel=True, want_cand=False, workspace=None, stream=None):
    """Allocate outputs and workspace with torch and run fs_fsb_prefill; tau is a float or
    [H] floats.  Returns (out or None, sel or None, cand or None, workspace)."""
    import torch
    sh = shape_of(k)
    ws_bytes = fs_fsb_workspace_bytes(sh, params, fsb)
    if ws_bytes == 0:
        raise FslError(FS_ERR_UNSUPPORTED, "fs_fsb_workspace_bytes")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    b, H, N, _ = k.shape
    out = torch.empty_like(k) if want_out else None
    sel = torch.empty(b, H, N, params.K, dtype=torch.int32, device=k.device) if want_sel else None
    cand = torch.empty(b, H, N, 2 * fsb.Wb, dtype=torch.int32, device=k.device) if want_cand else None
    fs_fsb_prefill(q, k, v, sigma, lam, tau, gain, out, sel, cand, workspace, params, fsb, stream)
    return out, sel, cand, workspace
