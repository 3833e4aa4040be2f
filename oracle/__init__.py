"""fp64 CPU oracle of FreeSolo's long-range branch (FS / FS-L).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the GPU library never
does, and the two share no code.  The arithmetic lives in ``fsl_oracle.c``
(plain C, fp64, one (sequence, head) per call); this file only marshals numpy
arrays into it and runs independent (sequence, head) pairs on a thread pool
(ctypes releases the GIL while the C code runs).

Page: "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
Extrapolation" (arXiv 2610.17191), Sec. 3.3 Eqs. 5-9 and App. D.2 Eq. 17; the
local branch of Sec. 3.2 (Eqs. 3-4) and the combination of Eq. 2.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfsl_oracle.so")
SOURCES = [os.path.join(_HERE, "fsl_oracle.c"), os.path.join(_HERE, "fsb_oracle.c")]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, *SOURCES, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("d", ctypes.c_int32), ("s", ctypes.c_int32),
                ("B", ctypes.c_int32), ("P", ctypes.c_int32), ("W", ctypes.c_int32),
                ("K", ctypes.c_int32), ("prune", ctypes.c_int32), ("sigma", ctypes.c_double),
                ("lambda_", ctypes.c_double), ("eps", ctypes.c_double)]


class _FsbCfg(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_double), ("Wb", ctypes.c_int32), ("c", ctypes.c_double)]


_lib = None


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_head.argtypes = [ctypes.POINTER(_Cfg), vp, vp, vp, vp, i64, i64, i64,
                                vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_head.restype = ctypes.c_int
    lib.oracle_cell_summaries.argtypes = [ctypes.POINTER(_Cfg), vp, vp, vp]
    lib.oracle_cell_summaries.restype = None
    lib.oracle_available_count.argtypes = [i64, ctypes.c_int32]
    lib.oracle_available_count.restype = i64
    lib.oracle_retained.argtypes = [ctypes.POINTER(_Cfg), i64, vp, vp, vp]
    lib.oracle_retained.restype = i64
    lib.oracle_cell_score.argtypes = [ctypes.POINTER(_Cfg), vp, vp, ctypes.c_double, i64, i64]
    lib.oracle_cell_score.restype = ctypes.c_double
    lib.oracle_cell_score_mag.argtypes = [ctypes.POINTER(_Cfg), vp, vp, ctypes.c_double, i64, i64]
    lib.oracle_cell_score_mag.restype = ctypes.c_double
    lib.oracle_readout.argtypes = [ctypes.POINTER(_Cfg), vp, vp, vp, vp, vp, i64, vp]
    lib.oracle_readout.restype = None
    lib.oracle_backward_head.argtypes = [ctypes.POINTER(_Cfg), vp, vp, vp, vp, vp, vp, i64, i64] + [vp] * 8
    lib.oracle_backward_head.restype = ctypes.c_int
    lib.oracle_fsb_chunks.argtypes = [i64, vp]
    lib.oracle_fsb_chunks.restype = ctypes.c_int32
    lib.oracle_fsb_forest.argtypes = [ctypes.POINTER(_Cfg), vp, vp, vp, i64, i64] + [vp] * 11
    lib.oracle_fsb_forest.restype = i64
    lib.oracle_fsb_node_priority.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_FsbCfg), vp, i64, vp,
                                             ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.oracle_fsb_node_priority.restype = ctypes.c_double
    lib.oracle_fsb_rerank_score.argtypes = [ctypes.POINTER(_Cfg), vp, vp, ctypes.c_double, i64, i64, vp]
    lib.oracle_fsb_rerank_score.restype = ctypes.c_double
    lib.oracle_fsb_head.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_FsbCfg), vp, vp, vp, vp, i64, i64] + [vp] * 7
    lib.oracle_fsb_head.restype = ctypes.c_int
    lib.oracle_local.argtypes = [i64, ctypes.c_int32, i64, ctypes.c_double, vp, vp, vp, ctypes.c_double, vp, i64, i64,
                                 vp]
    lib.oracle_local.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        # FSL_ORACLE_LIBRARY: an instrumented build of the same sources (the sanitizer test)
        _lib = _bind(os.environ.get("FSL_ORACLE_LIBRARY") or build())
    return _lib


class use_library:
    """Context manager: route this module's calls to another build of the oracle
    source (the mutation tests use it to run the pins against planted mistakes)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


@dataclass(frozen=True)
class Params:
    """Method parameters (defaults: the page's hyperparameters, App. A)."""
    s: int = 32
    B: int = 128
    P: int = 64
    W: int = 8
    K: int = 4
    prune: bool = True
    sigma: float = 4.0
    lam: float = 1.0
    eps: float = 1e-8

    def cfg(self, N: int, d: int) -> _Cfg:
        return _Cfg(N, d, self.s, self.B, self.P, self.W, self.K, int(self.prune),
                    self.sigma, self.lam, self.eps)


def _p(a):
    return None if a is None else a.ctypes.data


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def cell_summaries(k: np.ndarray, prm: Params = Params()):
    """Eq. 5 for one head: k [N, d] -> (kbar [N//s, d], a [N//s])."""
    k = _f64(k)
    N, d = k.shape
    M = N // prm.s
    kbar = np.zeros((M, d)); a = np.zeros(M)
    cfg = prm.cfg(N, d)
    _load().oracle_cell_summaries(ctypes.byref(cfg), _p(k), _p(kbar), _p(a))
    return kbar, a


def available_count(b_start: int, s: int = 32) -> int:
    """Eq. 6: |C_i| for a block starting at b_start."""
    return int(_load().oracle_available_count(b_start, s))


def retained(a: np.ndarray, n_avail: int, prm: Params = Params()):
    """Eq. 8 (or A = C for FS) for one block -> (ids ascending, gap_p)."""
    a = _f64(a)
    out = np.full(max(1, n_avail), -1, dtype=np.int32)
    gap = np.zeros(1)
    cfg = prm.cfg(len(a) * prm.s, 1)
    n = _load().oracle_retained(ctypes.byref(cfg), n_avail, _p(a), _p(out), _p(gap))
    return out[:n].copy(), float(gap[0])


def cell_score(q_i, kbar_c, a_c: float, i: int, c: int, prm: Params = Params()) -> float:
    """Eq. 7 for one (query, cell)."""
    q_i = _f64(q_i); kbar_c = _f64(kbar_c)
    cfg = prm.cfg(0, len(q_i))
    return float(_load().oracle_cell_score(ctypes.byref(cfg), _p(q_i), _p(kbar_c), float(a_c), i, c))


def cell_score_mag(q_i, kbar_c, a_c: float, i: int, c: int, prm: Params = Params()) -> float:
    """The size of the terms Eq. 7 sums for (query i, cell c); see fsl_oracle.h."""
    q_i = _f64(q_i); kbar_c = _f64(kbar_c)
    cfg = prm.cfg(0, len(q_i))
    return float(_load().oracle_cell_score_mag(ctypes.byref(cfg), _p(q_i), _p(kbar_c), float(a_c), i, c))


def readout(q_i, k, v, cells, g=None, prm: Params = Params()):
    """Eq. 9 + Eq. 17 for one query over a given selection `cells` (ids; -1 entries
    are ignored): q_i [d], k, v [N, d] -> o [d] (zero for an empty selection)."""
    q_i, k, v, g = _f64(q_i), _f64(k), _f64(v), _f64(g)
    T = np.ascontiguousarray([c for c in cells if c >= 0], dtype=np.int64)
    M = k.shape[0] // prm.s
    if np.any(T >= M):
        raise ValueError("selection names a cell past the last complete one")
    o = np.zeros(k.shape[1])
    cfg = prm.cfg(k.shape[0], k.shape[1])
    _load().oracle_readout(ctypes.byref(cfg), _p(q_i), _p(k), _p(v), _p(g), _p(T) if len(T) else None, len(T), _p(o))
    return o


def backward(q, k, v, sel, dout, g=None, prm: Params = Params(), i_lo: int = 0, i_hi: int | None = None,
             want_abs: bool = False):
    """Readout backward (Sec. 3.3 "Training") for one (sequence, head): the gradients of
    sum_i dout_i . o_i through the readout of the fixed selections sel [n, K] (queries i in
    [i_lo, i_hi)).  Returns dict dq [n, d], dk, dv [N, d], dg [d] (and the *_abs sizes)."""
    q, k, v, g, dout = _f64(q), _f64(k), _f64(v), _f64(g), _f64(dout)
    N, d = k.shape
    i_hi = N if i_hi is None else i_hi
    n = i_hi - i_lo
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    res = {"dq": np.zeros((n, d)), "dk": np.zeros((N, d)), "dv": np.zeros((N, d)), "dg": np.zeros(d)}
    if want_abs:
        res.update({"dq_abs": np.zeros((n, d)), "dk_abs": np.zeros((N, d)), "dv_abs": np.zeros((N, d)),
                    "dg_abs": np.zeros(d)})
    cfg = prm.cfg(N, d)
    rc = _load().oracle_backward_head(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), _p(sel), _p(dout), i_lo, i_hi,
                                      _p(res["dq"]), _p(res["dk"]), _p(res["dv"]), _p(res["dg"]),
                                      _p(res.get("dq_abs")), _p(res.get("dk_abs")), _p(res.get("dv_abs")),
                                      _p(res.get("dg_abs")))
    if rc != 0:
        raise ValueError("oracle_backward_head rejected its arguments")
    return res


def cap_for(N: int, prm: Params) -> int:
    M = N // prm.s
    return max(1, min(M, prm.P + prm.W) if prm.prune else M)


def head(q, k, v, g=None, prm: Params = Params(), i_lo: int = 0, i_hi: int | None = None,
         want_scores: bool = False, want_out: bool = True, want_summaries: bool = True):
    """The whole branch for one (sequence, head); q, k, v [N, d] (any float dtype).

    Returns a dict with kbar, a, retained [NB, cap], n_ret [NB], gap_p [NB],
    sel [n, K], gap_k [n], out [n, d] and optionally scores [n, cap], for the
    queries i in [i_lo, i_hi).  Blocks not touched by the range hold -1/NaN.
    """
    k = _f64(k)
    N, d = k.shape
    q = _f64(q) if q is not None else np.zeros((N, d))
    v = _f64(v) if v is not None else np.zeros((N, d))
    g = _f64(g)
    i_hi = N if i_hi is None else i_hi
    n = i_hi - i_lo
    M = N // prm.s
    NB = (N + prm.B - 1) // prm.B
    cap = cap_for(N, prm)
    res = {
        "kbar": np.zeros((M, d)) if want_summaries else None,
        "a": np.zeros(M) if want_summaries else None,
        "retained": np.full((max(NB, 1), cap), -1, dtype=np.int32),
        "n_ret": np.full(max(NB, 1), -1, dtype=np.int32),
        "gap_p": np.full(max(NB, 1), np.nan),
        "sel": np.full((n, prm.K), -1, dtype=np.int32),
        "gap_k": np.zeros(n),
        "out": np.zeros((n, d)) if want_out else None,
        "scores": np.full((n, cap), np.nan) if want_scores else None,
    }
    cfg = prm.cfg(N, d)
    rc = _load().oracle_head(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(g), i_lo, i_hi, cap,
                             _p(res["kbar"]), _p(res["a"]), _p(res["retained"]), _p(res["n_ret"]),
                             _p(res["gap_p"]), _p(res["sel"]), _p(res["gap_k"]), _p(res["out"]),
                             _p(res["scores"]))
    if rc != 0:
        raise ValueError("oracle_head rejected its arguments")
    return res


def batch(q, k, v, g=None, prm: Params = Params(), heads=None, i_lo: int = 0, i_hi: int | None = None,
          threads: int | None = None, want_out: bool = True):
    """Run `head` over (b, h) pairs of [batch, H, N, d] arrays on a thread pool.

    `g` is [H, d] or None.  Returns {(b, h): result}.
    """
    Bt, H = k.shape[0], k.shape[1]
    pairs = heads if heads is not None else [(b, h) for b in range(Bt) for h in range(H)]

    def one(p):
        b, h = p
        return p, head(None if q is None else q[b, h], k[b, h], None if v is None else v[b, h],
                       None if g is None else g[h], prm, i_lo, i_hi, want_out=want_out)

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        return dict(ex.map(one, pairs))


def local(q, k, v, w: int = 512, rope_base: float = 10000.0, alpha: float = 0.0, o_lr=None, i_lo: int = 0,
          i_hi: int | None = None):
    """Local branch (Sec. 3.2, Eqs. 3-4) for one head, plus alpha * o_lr (Eq. 2) when o_lr
    [(i_hi - i_lo), d] is given: q, k, v [N, d] -> out [(i_hi - i_lo), d]."""
    q, k, v, o_lr = _f64(q), _f64(k), _f64(v), _f64(o_lr)
    N, d = k.shape
    i_hi = N if i_hi is None else i_hi
    out = np.zeros((i_hi - i_lo, d))
    rc = _load().oracle_local(N, d, w, rope_base, _p(q), _p(k), _p(v), alpha, _p(o_lr), i_lo, i_hi, _p(out))
    if rc != 0:
        raise ValueError("oracle_local rejected its arguments")
    return out


# ------------------------------------------------------------------ FS-B (Sec. 3.4; App. E.1) ----

@dataclass(frozen=True)
class FsbParams:
    """FS-B parameters: the second forest's norm threshold tau (Eq. 10), the beam width W^b and
    the radius weight c of Eq. 11 (the page uses W^b = 16, c = 8)."""
    tau: float = 0.0
    Wb: int = 16
    c: float = 8.0

    def cfg(self) -> _FsbCfg:
        return _FsbCfg(self.tau, self.Wb, self.c)


def fsb_chunks(M: int) -> list:
    """Eq. 18: the chunk sizes of M admitted cells, largest first."""
    sizes = np.zeros(64, dtype=np.int64)
    r = _load().oracle_fsb_chunks(M, _p(sizes))
    return [int(x) for x in sizes[:r]]


def fsb_forest(kbar, a, cells, prm: Params = Params()):
    """One forest (App. E.1) over the admitted `cells` (arrival order); returns a dict of node
    arrays (count, cell, left, right, minid, mu, rho, A, pmin), the root and the smallest
    median-split gap."""
    kbar, a = _f64(kbar), _f64(a)
    cells = np.ascontiguousarray(cells, dtype=np.int64)
    M, d = len(cells), kbar.shape[1]
    cap = max(1, 2 * M + 1)
    out = {x: np.zeros(cap, dtype=np.int64) for x in ("count", "cell", "left", "right", "minid")}
    out.update({x: np.zeros(cap) for x in ("rho", "A", "pmin")})
    out["mu"] = np.zeros((cap, d))
    n_nodes = np.zeros(1, dtype=np.int64)
    gap = np.full(1, np.inf)
    cfg = prm.cfg(kbar.shape[0] * prm.s, d)
    root = _load().oracle_fsb_forest(ctypes.byref(cfg), _p(kbar), _p(a), _p(cells) if M else None, M, cap,
                                     _p(out["count"]), _p(out["cell"]), _p(out["left"]), _p(out["right"]),
                                     _p(out["minid"]), _p(out["mu"]), _p(out["rho"]), _p(out["A"]), _p(out["pmin"]),
                                     _p(n_nodes), _p(gap))
    n = int(n_nodes[0]) if root >= 0 else 0
    res = {x: y[:n].copy() for x, y in out.items()}
    res["root"] = int(root)
    res["min_split_gap"] = float(gap[0])
    return res


def fsb_node_priority(q_i, i: int, mu, rho: float, A: float, pmin: float, prm: Params = Params(),
                      fb: FsbParams = FsbParams()) -> float:
    """Eq. 11 for one node summary."""
    q_i, mu = _f64(q_i), _f64(mu)
    cfg, fc = prm.cfg(0, len(q_i)), fb.cfg()
    return float(_load().oracle_fsb_node_priority(ctypes.byref(cfg), ctypes.byref(fc), _p(q_i), i, _p(mu),
                                                  float(rho), float(A), float(pmin)))


def fsb_rerank_score(q_i, k, a_c: float, i: int, c: int, prm: Params = Params()):
    """Eq. 12 for query i and cell c -> (score, size of its terms)."""
    q_i, k = _f64(q_i), _f64(k)
    mag = np.zeros(1)
    cfg = prm.cfg(k.shape[0], k.shape[1])
    r = _load().oracle_fsb_rerank_score(ctypes.byref(cfg), _p(q_i), _p(k), float(a_c), i, c, _p(mag))
    return float(r), float(mag[0])


def fsb_head(q, k, v, g=None, prm: Params = Params(), fb: FsbParams = FsbParams(), i_lo: int = 0,
             i_hi: int | None = None, want_out: bool = True):
    """FS-B for one (sequence, head): dict with sel [n, K], cand [n, 2 W^b], n_cand [n],
    gap_beam, gap_rerank, gap_split [n], out [n, d], and the cell summaries kbar, a."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    N, d = k.shape
    i_hi = N if i_hi is None else i_hi
    n = i_hi - i_lo
    res = {"sel": np.full((n, prm.K), -1, dtype=np.int32), "cand": np.full((n, 2 * fb.Wb), -1, dtype=np.int32),
           "n_cand": np.zeros(n, dtype=np.int32), "gap_beam": np.zeros(n), "gap_rerank": np.zeros(n),
           "gap_split": np.zeros(n), "out": np.zeros((n, d)) if want_out else None}
    cfg, fc = prm.cfg(N, d), fb.cfg()
    rc = _load().oracle_fsb_head(ctypes.byref(cfg), ctypes.byref(fc), _p(q), _p(k), _p(v), _p(g), i_lo, i_hi,
                                 _p(res["sel"]), _p(res["cand"]), _p(res["n_cand"]), _p(res["gap_beam"]),
                                 _p(res["gap_rerank"]), _p(res["gap_split"]), _p(res["out"]))
    if rc != 0:
        raise ValueError("oracle_fsb_head rejected its arguments")
    res["kbar"], res["a"] = cell_summaries(k, prm)
    return res
