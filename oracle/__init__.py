"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it, and the
two share no code: the oracle is a plain token-sequential C implementation in
double precision (``gdn_oracle.c``) plus the fp64 chunkwise rewrite in
``chunked.py`` that pins the chunk algebra.

Source of the method: SANA-Streaming pages -- the Korean review, section 1 (GDN
keeps a fixed-size state updated recursively) and the Chinese summary, "Method
steps" step 2 (forward scan carrying the previous chunk's cache, plus a
backward scan inside the chunk).  The update itself is the published Gated
DeltaNet rule, which the pages name but do not print:

    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale * S_t q_t
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_variants = {}

DEFAULT_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lpthread", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.gdn_oracle_scan.argtypes = [i64, i64, i64, i64, i64,
                                    dp, dp, dp, dp, dp, dp,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                    dp, dp, ctypes.c_int, i64]
    lib.gdn_oracle_scan.restype = ctypes.c_int
    lib.gdn_oracle_backward.argtypes = [i64, i64, i64, i64, i64,
                                        dp, dp, dp, dp, dp, dp, dp, dp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                        dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.gdn_oracle_backward.restype = ctypes.c_int
    return lib


def _load(path=None):
    """The default oracle library, or (for the pin tests' planted-mistake checks) another build."""
    global _lib
    if path is not None:
        if path not in _variants:
            _variants[path] = _bind(path)
        return _variants[path]
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB)
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def scan(q, k, v, a, beta, S0=None, *, reverse=False, l2norm=True, eps=DEFAULT_EPS,
         scale=1.0, threads=None, row_block=16, lib=None):
    """Token-sequential gated delta rule over all streams and heads.

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; a, beta: [B, T, H]; S0: [B, H, Dv, Dk] or None.
    Returns (o [B, T, H, Dv], S_final [B, H, Dv, Dk]) in float64.  ``reverse``
    scans t = T-1 .. 0 from S0 (zero when None).  ``lib`` names another build of
    ``gdn_oracle.c`` (used only by the tests that plant mistakes in a copy).
    """
    q, k, v, a, beta = (_f64(x) for x in (q, k, v, a, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    assert a.shape == (B, T, H) and beta.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, Dv, Dk)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    S_final = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    rc = _load(lib).gdn_oracle_scan(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta),
                                 _ptr(S0), int(bool(reverse)), int(bool(l2norm)), float(eps),
                                 float(scale), _ptr(o), _ptr(S_final),
                                 int(threads or default_threads()), int(row_block))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_scan failed with code {rc}")
    return o, S_final


def forward(q, k, v, a, beta, S0=None, **kw):
    """Causal forward scan from the carried state S0 (zero when None)."""
    return scan(q, k, v, a, beta, S0, reverse=False, **kw)


def reverse(q, k, v, a, beta, **kw):
    """Intra-chunk backward scan: starts from a zero state at the chunk end."""
    return scan(q, k, v, a, beta, None, reverse=True, **kw)


def backward(q, k, v, a, beta, dO, S0=None, dS_final=None, *, reverse=False, l2norm=True,
             eps=DEFAULT_EPS, scale=1.0, threads=None, lib=None):
    """Gradients of ``scan`` (reverse-mode through the per-token rule, fp64).

    dO: gradient of the loss with respect to o [B, T, H, Dv]; dS_final: with respect to the
    final state [B, H, Dv, Dk] (None = zero).  Returns a dict with dq, dk [B, T, H, Dk],
    dv [B, T, H, Dv], da, dbeta [B, T, H] and dS0 [B, H, Dv, Dk].  Training over streaming
    chunks (the Chinese summary, "Method steps") needs this pass; the pages print no
    formula for it, so it is the derivative of the recurrence itself.
    """
    q, k, v, a, beta, dO = (_f64(x) for x in (q, k, v, a, beta, dO))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv) and dO.shape == (B, T, H, Dv)
    assert a.shape == (B, T, H) and beta.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    dS_final = None if dS_final is None else _f64(dS_final)
    for x in (S0, dS_final):
        if x is not None:
            assert x.shape == (B, H, Dv, Dk)
    out = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)), "dv": np.zeros((B, T, H, Dv)),
           "da": np.zeros((B, T, H)), "dbeta": np.zeros((B, T, H)), "dS0": np.zeros((B, H, Dv, Dk))}
    rc = _load(lib).gdn_oracle_backward(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta),
                                     _ptr(S0), _ptr(dO), _ptr(dS_final), int(bool(reverse)),
                                     int(bool(l2norm)), float(eps), float(scale),
                                     _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["da"]),
                                     _ptr(out["dbeta"]), _ptr(out["dS0"]), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_backward failed with code {rc}")
    return out
