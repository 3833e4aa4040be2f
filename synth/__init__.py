"""Seeded synthetic inputs for the long-range branch workloads.

This module draws the query, key and value tensors (and optional RMSNorm gains)
that both the GPU path and the fp64 CPU oracle consume.  It contains none of the
attention method's arithmetic.

Recipe (every value is a pure function of the seed, a stream id and a flat index,
so any (batch, head, position) slice can be regenerated on its own):

* q, k, v feature values: standard normal per feature (streams 1, 2, 3), flat
  index ``((b * H + h) * N + n) * d + f`` over the logical length N.
* keys only: each key row is multiplied by ``exp(sigma_ln * xi)`` with
  ``xi ~ N(0, 1)`` drawn per token (stream 4), i.e. a lognormal(0, sigma_ln)
  factor, and, for exactly ``round(needle_frac * N)`` distinct positions per
  (batch, head), by ``needle_scale`` (the "needles").  The needle positions are
  the ones whose 64-bit draw on stream 5 is smallest, a uniform random subset.
* values are computed in fp64, rounded to fp32, and for bf16 workloads rounded
  again (nearest-even) to bf16.
* optional gains: uniform on [0.5, 1.5) per (head, feature), stream 6.
* upstream gradients dout (the loss gradient of a branch output, for the readout
  backward): standard normal per feature, stream 7, flat index as for q.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_SRC_PATH = os.path.join(_HERE, "gen.c")

STREAM_Q, STREAM_K, STREAM_V, STREAM_KSCALE, STREAM_NEEDLE, STREAM_GAIN, STREAM_DOUT = 1, 2, 3, 4, 5, 6, 7


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC_PATH, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        u64 = ctypes.c_uint64
        lib.synth_bits.argtypes = [u64, u64, u64, u64, ctypes.c_void_p]
        lib.synth_bits.restype = None
        lib.synth_normal_f64.argtypes = [u64, u64, u64, u64, ctypes.c_void_p]
        lib.synth_normal_f64.restype = None
        lib.synth_rows.argtypes = [u64, u64, u64, u64, ctypes.c_uint32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_rows.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def bits(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _load().synth_bits(seed, stream, start, count, _ptr(out))
    return out


def normals(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    _load().synth_normal_f64(seed, stream, start, count, _ptr(out))
    return out


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic long-range workload."""
    batch: int
    H: int
    N: int            # logical sequence length (prefix plus any decode steps)
    d: int
    dtype: str        # "f32" or "bf16"
    seed: int
    needle_frac: float = 0.0
    sigma_ln: float = 0.5
    needle_scale: float = 4.0
    name: str = field(default="", compare=False)

    @property
    def n_needles(self) -> int:
        return int(round(self.needle_frac * self.N))


def needle_positions(w: Workload, b: int, h: int) -> np.ndarray:
    """Sorted needle token positions of sequence b, head h."""
    m = w.n_needles
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    draws = bits(w.seed, STREAM_NEEDLE, (b * w.H + h) * w.N, w.N)
    # stable ordering by (draw, position): a uniform random m-subset
    order = np.lexsort((np.arange(w.N), draws))
    return np.sort(order[:m]).astype(np.int64)


def key_row_scale(w: Workload, b: int, h: int, n0: int, n1: int,
                  needles: np.ndarray | None = None) -> np.ndarray:
    """fp64 multiplier of key rows n0..n1-1 of (b, h)."""
    xi = normals(w.seed, STREAM_KSCALE, (b * w.H + h) * w.N + n0, n1 - n0)
    sc = np.exp(w.sigma_ln * xi)
    if w.n_needles > 0:
        pos = needle_positions(w, b, h) if needles is None else needles
        sel = pos[(pos >= n0) & (pos < n1)] - n0
        sc[sel] *= w.needle_scale
    return sc


def _storage_dtype(dtype: str):
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16  # bf16 bit patterns
    raise ValueError("dtype must be 'f32' or 'bf16'")


def tensor(w: Workload, which: str, n0: int = 0, n1: int | None = None,
           heads: list[tuple[int, int]] | None = None, threads: int | None = None) -> np.ndarray:
    """One of 'q', 'k', 'v', 'dout' for positions [n0, n1).

    Returns a C-contiguous array [batch, H, n1-n0, d] (or [len(heads), n1-n0, d]
    when `heads` lists (b, h) pairs) of float32, or of uint16 bf16 bit patterns.
    """
    n1 = w.N if n1 is None else n1
    stream = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V, "dout": STREAM_DOUT}[which]
    pairs = heads if heads is not None else [(b, h) for b in range(w.batch) for h in range(w.H)]
    rows = n1 - n0
    st = _storage_dtype(w.dtype)
    out = np.empty((len(pairs), rows, w.d), dtype=st)
    lib = _load()
    chunk = 4096

    def work(job):
        slot, (b, h), r0 = job
        r1 = min(rows, r0 + chunk)
        scale = None
        if which == "k":
            scale = np.ascontiguousarray(key_row_scale(w, b, h, n0 + r0, n0 + r1, needles_of[(b, h)]))
        view = out[slot, r0:r1]
        row0 = (b * w.H + h) * w.N + n0 + r0
        if w.dtype == "bf16":
            lib.synth_rows(w.seed, stream, row0, r1 - r0, w.d, _ptr(scale), None, _ptr(view))
        else:
            lib.synth_rows(w.seed, stream, row0, r1 - r0, w.d, _ptr(scale), _ptr(view), None)

    needles_of = {}
    if which == "k":
        for p in pairs:
            needles_of[p] = needle_positions(w, *p) if w.n_needles > 0 else None
    jobs = [(slot, p, r0) for slot, p in enumerate(pairs) for r0 in range(0, rows, chunk)]
    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        list(ex.map(work, jobs))
    if heads is None:
        out = out.reshape(w.batch, w.H, rows, w.d)
    return out


def gains(seed: int, H: int, d: int) -> np.ndarray:
    """RMSNorm gains in [0.5, 1.5), float32 [H, d]."""
    u = (bits(seed, STREAM_GAIN, 0, H * d) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return (0.5 + u).astype(np.float32).reshape(H, d)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of generated storage (fp32, or bf16 bit patterns) to fp64."""
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# The workloads the path is measured and checked on (seeded, synthetic).
WORKLOADS = {
    "small_fs_equiv": Workload(batch=1, H=2, N=1024, d=64, dtype="f32", seed=1, needle_frac=0.0,
                               name="FS-L prefill b1 H2 d64 N1024 f32 (FS-L == FS)"),
    "prefill_4k": Workload(batch=1, H=8, N=4096, d=64, dtype="f32", seed=2, needle_frac=0.01,
                           name="FS-L prefill b1 H8 d64 N4096 f32, 1% needles"),
    "prefill_16k": Workload(batch=4, H=16, N=16384, d=128, dtype="bf16", seed=3, needle_frac=0.005,
                            name="FS-L prefill b4 H16 d128 N16384 bf16, 0.5% needles"),
    "fs_32k": Workload(batch=1, H=16, N=32768, d=128, dtype="bf16", seed=4, needle_frac=0.005,
                       name="FS prefill b1 H16 d128 N32768 bf16, 0.5% needles"),
    "train_4k": Workload(batch=16, H=16, N=4096, d=64, dtype="bf16", seed=6, needle_frac=0.005,
                         name="FS-L readout backward b16 H16 d64 N4096 bf16 (one GPU's share of a 524,288-token "
                              "training step of the 16-head, 64-wide attention), 0.5% needles"),
    "decode_256k": Workload(batch=32, H=8, N=262144 + 128, d=128, dtype="bf16", seed=5, needle_frac=0.005,
                            name="FS-L decode b32 H8 d128, 262144-token prefix + 128 steps, bf16"),
}
