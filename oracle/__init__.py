"""fp64 CPU oracle for the Simple GLA mixer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and this package imports nothing
from the product.

The arithmetic lives in ``gla_oracle.c`` (plain per-token recurrence in fp64,
see its header for the passages of the Laplace 3B post it follows).  This
module only builds that file with the host C compiler and marshals numpy
arrays to it.

Parity status of each function (what pins it is in tests/test_oracle.py):
  fwd     pinned: lambda=1 causal linear attention, lambda=0 (q.k)v, the
          quadratic decay-masked form, chunked == recurrent, split/resume.
  bwd     pinned: central finite differences, fp64 autograd of the quadratic
          form, and the (t+1)(q.dq - k.dk) identity for dlambda.
  decode  pinned: k decode steps == forward over the same k tokens, and the
          lambda=0 / lambda=1 closed forms.
  epilogue  pinned: closed forms -- a constant head vector normalises to
          sign * w of its tier, a one-hot value with a gate of sigmoid(ln 3)
          = 3/4 gives the 7/4 channel ratio, a = 0 gives the half skip,
          silu(ln 3) = (3/4) ln 3, a zero vector stays zero (eps > 0).
  conv1d, conv1d_decode  pinned: fp64 torch grouped conv1d (the library's
          cross-correlation with K-1 left padding, or the window prepended),
          the impulse response w reversed through silu, decode steps == prefill,
          split/resume through the window, the window carry itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgla_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile gla_oracle.c into oracle/libgla_oracle.so with gcc + OpenMP."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    i = ctypes.c_int
    lib.gla_oracle_fwd.argtypes = [i, i, i, i, i, _D, _D, _D, _D, _D,
                                   ctypes.c_double, _D, _D, i]
    lib.gla_oracle_bwd.argtypes = [i, i, i, i, i, _D, _D, _D, _D, _D,
                                   ctypes.c_double, _D, _D, _D, _D, _D,
                                   _D, _D, i]
    lib.gla_oracle_decode.argtypes = [i, i, i, i, _D, _D, _D, _D, _D,
                                      ctypes.c_double, _D, i]
    lib.gla_oracle_epilogue.argtypes = [i, i, i, i, _D, _D, _D, _D, _D, _D, _D,
                                        ctypes.POINTER(ctypes.c_int), i, ctypes.c_double, _D, i]
    lib.gla_oracle_conv1d.argtypes = [i, i, i, i, _D, _D, _D, _D, _D, _D, i]
    lib.gla_oracle_conv1d_decode.argtypes = [i, i, i, _D, _D, _D, _D, _D, i]
    for f in (lib.gla_oracle_fwd, lib.gla_oracle_bwd, lib.gla_oracle_decode,
              lib.gla_oracle_epilogue, lib.gla_oracle_conv1d, lib.gla_oracle_conv1d_decode):
        f.restype = ctypes.c_int
    lib.gla_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
            ):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile an edited copy of the oracle source (used by the tests that plant
    a mistake in the oracle to show the pins catch it) and return its functions
    as an object with fwd/bwd/decode methods."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-o", out_path, src], check=True)
    return _Variant(_bind(ctypes.CDLL(out_path)))


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def max_threads() -> int:
    return int(_load().gla_oracle_max_threads())


def fwd(q, k, v, lam, S0=None, scale=1.0, nthreads=0, _lib_=None):
    """q,k [B,T,H,dk], v [B,T,H,dv], lam [H] -> (o [B,T,H,dv], S_final [B,H,dk,dv])."""
    q, k, v, lam, S0 = map(_f64, (q, k, v, lam, S0))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H) and lam.shape == (H,)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    rc = (_lib_ or _load()).gla_oracle_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(lam),
                                _p(S0), float(scale), _p(o), _p(S), int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_fwd failed")
    return o, S


def bwd(q, k, v, lam, d_o, S0=None, dS_T=None, scale=1.0, nthreads=0, _lib_=None):
    """Gradients of <do,o> + <dS_T,S_final>: returns dq, dk, dv, dlambda[H], dS0."""
    q, k, v, lam, d_o, S0, dS_T = map(_f64, (q, k, v, lam, d_o, S0, dS_T))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert d_o.shape == v.shape
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dlam = np.zeros(H)
    dS0 = np.zeros((B, H, dk, dv))
    rc = (_lib_ or _load()).gla_oracle_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(lam),
                                _p(S0), float(scale), _p(d_o), _p(dS_T), _p(dq),
                                _p(dkk), _p(dvv), _p(dlam), _p(dS0), int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_bwd failed")
    return dq, dkk, dvv, dlam, dS0


def decode(q, k, v, lam, S, scale=1.0, nthreads=0, _lib_=None):
    """One decode step: q,k [N,H,dk], v [N,H,dv], S [N,H,dk,dv] -> (o, S_new)."""
    q, k, v, lam = map(_f64, (q, k, v, lam))
    S = np.array(S, dtype=np.float64, copy=True, order="C")
    N, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv))
    rc = (_lib_ or _load()).gla_oracle_decode(N, H, dk, dv, _p(q), _p(k), _p(v), _p(lam),
                                   _p(S), float(scale), _p(o), int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_decode failed")
    return o, S


def epilogue(q, k, v, o, g, a, w, tier, eps=1e-6, nthreads=0, _lib_=None):
    """Mixer epilogue: q,k [..., H, dk]; v, o, g [..., H, dv]; a [H, dk] or None (a = 0);
    w [n_tiers, dv]; tier [H] ints -> y [..., H, dv]."""
    q, k, v, o, g, w = map(_f64, (q, k, v, o, g, w))
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    M = int(np.prod(q.shape[:-2]))
    ap = None if a is None else _f64(a)
    t = np.ascontiguousarray(np.asarray(tier, dtype=np.int32))
    y = np.zeros(v.shape)
    rc = (_lib_ or _load()).gla_oracle_epilogue(
        M, H, dk, dv, _p(q), _p(k), _p(v), _p(o), _p(g), _p(ap) if ap is not None else None, _p(w),
        t.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), int(w.shape[0]), float(eps), _p(y), int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_epilogue failed")
    return y


def conv1d(x, w, bias=None, win=None, nthreads=0, _lib_=None):
    """Depth-wise causal conv + SiLU: x [B, T, D], w [D, K], bias [D] or None,
    win [B, K, D] or None (zeros) -> (y [B, T, D], window after the last token [B, K, D])."""
    x, w, bias, win = map(_f64, (x, w, bias, win))
    B, T, D = x.shape
    K = w.shape[1]
    y = np.zeros((B, T, D))
    wo = np.zeros((B, K, D))
    rc = (_lib_ or _load()).gla_oracle_conv1d(B, T, D, K, _p(x), _p(w), _p(bias), _p(win), _p(y), _p(wo),
                                              int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_conv1d failed")
    return y, wo


def conv1d_decode(x, w, bias, win, nthreads=0, _lib_=None):
    """One token per sequence: x [N, D], win [N, K, D] -> (y [N, D], new window)."""
    x, w, bias = map(_f64, (x, w, bias))
    win = np.array(win, dtype=np.float64, copy=True, order="C")
    N, D = x.shape
    K = w.shape[1]
    y = np.zeros((N, D))
    rc = (_lib_ or _load()).gla_oracle_conv1d_decode(N, D, K, _p(x), _p(w), _p(bias), _p(win), _p(y),
                                                     int(nthreads))
    if rc != 0:
        raise RuntimeError("gla_oracle_conv1d_decode failed")
    return y, win


class _Variant:
    def __init__(self, lib):
        self.lib = lib

    def fwd(self, *a, **kw):
        return fwd(*a, _lib_=self.lib, **kw)

    def bwd(self, *a, **kw):
        return bwd(*a, _lib_=self.lib, **kw)

    def decode(self, *a, **kw):
        return decode(*a, _lib_=self.lib, **kw)

    def epilogue(self, *a, **kw):
        return epilogue(*a, _lib_=self.lib, **kw)

    def conv1d(self, *a, **kw):
        return conv1d(*a, _lib_=self.lib, **kw)

    def conv1d_decode(self, *a, **kw):
        return conv1d_decode(*a, _lib_=self.lib, **kw)
