"""ctypes binding of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module to compute expected values.  The GPU library
never imports it, and it never imports the GPU library.

The oracle computes the hybrid layer of Lizard (gist.science technical summary of
paper 2507.09025, Methodology sections A.1 and A.2) token by token in double
precision; ``oracle.c`` lists the readings it takes where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

PART_GLA = 1
PART_SWA = 2
PART_BOTH = 3

# Gate layouts (the same codes as the library's glah_gate_kind).  The scalar
# ones are the fixed/scalar-decay variants the pages list beside GLA (a per-token
# scalar as in Mamba-2, a fixed per-head decay as in RetNet: "LT2" technical
# summary, 2.1 architecture variants; "systematic analysis of hybrid linear
# attention", evaluated models): a log-gate equal for every feature.
GATE_LOGITS = 0     # [B,H,L,f] logits
GATE_LOG = 1        # [B,H,L,f] log Gamma
GATE_LOG_TOKEN = 2  # [B,H,L] log Gamma of each token, every feature
GATE_LOG_HEAD = 3   # [H] fixed log Gamma of each head, every token and feature


def _gate_per_feature(g, kind, B, H, L, f):
    """Per-feature gates [B,H,L,f] (L = None: decode [B,H,f]) and whether they
    are log-gates, for gate layout ``kind``: scalar gates are broadcast."""
    g = np.asarray(g, dtype=np.float64)
    if kind in (GATE_LOGITS, GATE_LOG):
        return g, kind == GATE_LOG
    if kind == GATE_LOG_TOKEN:
        shape = (B, H, f) if L is None else (B, H, L, f)
        return np.ascontiguousarray(np.broadcast_to(g[..., None], shape)), True
    if kind == GATE_LOG_HEAD:
        shape = (B, H, f) if L is None else (B, H, L, f)
        h = g.reshape(1, H, 1) if L is None else g.reshape(1, H, 1, 1)
        return np.ascontiguousarray(np.broadcast_to(h, shape)), True
    raise ValueError("unknown gate kind %r" % (kind,))

_lock = threading.Lock()
_default = None


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into a shared library with gcc (-O2, OpenMP)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` when missing or stale."""
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """One loaded build of the oracle library (the default build, or a test variant)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_layer_fwd.argtypes = [i] * 8 + [ctypes.c_double, i, i] + [dp] * 10
        lib.oracle_layer_fwd.restype = i
        lib.oracle_decode_step.argtypes = ([i] * 7 + [ctypes.c_double, i, i] + [dp] * 10
                                           + [ctypes.POINTER(ctypes.c_longlong), dp])
        lib.oracle_decode_step.restype = i
        lib.oracle_num_threads.restype = i
        lib.oracle_set_num_threads.argtypes = [i]
        self.lib = lib

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def layer_fwd(self, q, k, v, g, wq, wk, meta, *, window, scale=None, gate_is_log=False,
                  parts=PART_BOTH, state_in=None, return_state=False, gate_kind=None):
        """Hybrid layer forward over whole sequences.

        q, k: [B,H,L,d]; v: [B,H,L,dv]; g: [B,H,L,f] gate logits (log-gates when
        ``gate_is_log``; other layouts with ``gate_kind``); wq, wk: [H,d,f/2];
        meta: [H,M] or None; state_in: [B,H,f,dv] or None.  Returns o [B,H,L,dv]
        (and the final state when ``return_state``).
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, L, d = q.shape
        dv = v.shape[-1]
        if parts & PART_GLA:
            wq, wk = _f64(wq), _f64(wk)
            f = 2 * wq.shape[-1]
            kind = gate_kind if gate_kind is not None else (GATE_LOG if gate_is_log else GATE_LOGITS)
            g, gate_is_log = _gate_per_feature(g, kind, B, H, L, f)
            g = _f64(g)
        else:
            g = wq = wk = None
            f = state_in.shape[-2] if state_in is not None else 2
        meta = _f64(meta) if meta is not None else None
        n_meta = 0 if meta is None else meta.shape[-1]
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        state_in = _f64(state_in)
        o = np.zeros((B, H, L, dv), dtype=np.float64)
        st = np.zeros((B, H, f, dv), dtype=np.float64) if return_state else None
        rc = self.lib.oracle_layer_fwd(B, H, L, d, dv, f, int(window), n_meta, float(scale),
                                       int(bool(gate_is_log)), int(parts),
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(wq), _ptr(wk),
                                       _ptr(meta), _ptr(state_in), _ptr(st), _ptr(o))
        if rc != 0:
            raise ValueError("oracle_layer_fwd rejected its arguments")
        return (o, st) if return_state else o

    def decode_step(self, q, k, v, g, wq, wk, meta, state, kcache, vcache, pos, *, window,
                    scale=None, gate_is_log=False, parts=PART_BOTH, gate_kind=None):
        """One decode step; ``state``, ``kcache`` and ``vcache`` (float64,
        C-contiguous) are updated in place.  q,k: [B,H,d]; v: [B,H,dv]; g: [B,H,f];
        pos: [B] ints (tokens already consumed).  Returns o [B,H,dv]."""
        for name, a in (("state", state), ("kcache", kcache), ("vcache", vcache)):
            if a.dtype != np.float64 or not a.flags.c_contiguous:
                raise TypeError(name + " must be a C-contiguous float64 array (updated in place)")
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, d = q.shape
        dv = v.shape[-1]
        f = state.shape[-2]
        kind = gate_kind if gate_kind is not None else (GATE_LOG if gate_is_log else GATE_LOGITS)
        g, gate_is_log = _gate_per_feature(g, kind, B, H, None, f)
        g, wq, wk = _f64(g), _f64(wq), _f64(wk)
        meta = _f64(meta) if meta is not None else None
        n_meta = 0 if meta is None else meta.shape[-1]
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        pos = np.ascontiguousarray(pos, dtype=np.int64)
        o = np.zeros((B, H, dv), dtype=np.float64)
        rc = self.lib.oracle_decode_step(B, H, d, dv, f, int(window), n_meta, float(scale),
                                         int(bool(gate_is_log)), int(parts),
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(wq), _ptr(wk),
                                         _ptr(meta), _ptr(state), _ptr(kcache), _ptr(vcache),
                                         pos.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)), _ptr(o))
        if rc != 0:
            raise ValueError("oracle_decode_step rejected its arguments")
        return o


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use when missing)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def layer_fwd(*args, **kw):
    return default().layer_fwd(*args, **kw)


def decode_step(*args, **kw):
    return default().decode_step(*args, **kw)


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)
