"""fp64 chunkwise form of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

This pins the algebra a chunked GPU kernel relies on ("chunked equals
token-sequential").  It is derived here from the per-token rule (SANA-Streaming
pages: Korean review section 1 defines GDN as a recursive fixed-size state; the
Chinese summary, "Method steps" step 4, names a fused kernel that works chunk by
chunk).  Within a chunk of C tokens that starts from state S0, with
g_t = sum_{s<=t} log a_s and gamma_t = exp(g_t):

    L[t, s]  = beta_t exp(g_t - g_s) (k_t . k_s)            s < t   (strictly lower)
    U        = (I + L)^{-1} (diag(beta) V - diag(beta gamma) K S0^T)
    O        = diag(gamma) Q S0^T + (M o (Q K^T)) U,   M[t, s] = exp(g_t - g_s), s <= t
    S_C      = gamma_C S0 + U^T diag(exp(g_C - g)) K

(rows u_t of U satisfy S_t = a_t S_{t-1} + u_t k_t^T).  Every exponent is <= 0.
Nothing here is shared with the GPU path; it exists so the CPU tests can check
that the rewrite equals the plain per-token definition in ``gdn_oracle.c``.
"""
from __future__ import annotations

import numpy as np


def _normalise(x, on, eps):
    if not on:
        return x
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def chunked_scan_head(q, k, v, a, beta, S0, C, *, l2norm=True, eps=1e-6, scale=1.0):
    """One (stream, head): q, k [T, Dk], v [T, Dv], a, beta [T], S0 [Dv, Dk] -> (o, S_T).

    Processes tokens 0..T-1 in chunks of C (the last chunk may be shorter).
    """
    q = _normalise(np.asarray(q, np.float64), l2norm, eps)
    k = _normalise(np.asarray(k, np.float64), l2norm, eps)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]), dtype=np.float64)
    for c0 in range(0, T, C):
        c1 = min(c0 + C, T)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        bt = beta[c0:c1]
        g = np.cumsum(np.log(a[c0:c1]))
        gam = np.exp(g)
        n = c1 - c0
        diff = g[:, None] - g[None, :]
        lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
        lower = np.tril(np.ones((n, n), dtype=bool), 0)
        decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        L = np.where(lower_strict, bt[:, None] * decay * (K @ K.T), 0.0)
        R = bt[:, None] * V - (bt * gam)[:, None] * (K @ S.T)
        U = np.linalg.solve(np.eye(n) + L, R)
        o[c0:c1] = scale * (gam[:, None] * (Q @ S.T) + (decay * (Q @ K.T)) @ U)
        w = np.exp(g[-1] - g)
        S = gam[-1] * S + U.T @ (w[:, None] * K)
    return o, S


def chunked_scan(q, k, v, a, beta, S0=None, *, C=64, reverse=False, **kw):
    """All streams and heads; same array layout as ``oracle.scan``."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    a, beta = np.asarray(a, np.float64), np.asarray(beta, np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    S_out = np.zeros((B, H, Dv, Dk))
    sl = slice(None, None, -1) if reverse else slice(None)
    for b in range(B):
        for h in range(H):
            S0bh = np.zeros((Dv, Dk)) if S0 is None else S0[b, h]
            ob, Sb = chunked_scan_head(q[b, sl, h], k[b, sl, h], v[b, sl, h], a[b, sl, h],
                                       beta[b, sl, h], S0bh, C, **kw)
            o[b, :, h] = ob[sl]
            S_out[b, h] = Sb
    return o, S_out
