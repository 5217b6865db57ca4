"""Numpy fp64 twin of the C oracle, for tiny inputs (test infrastructure only).

TEST INFRASTRUCTURE: only the tests may import this module. It is a second,
independent transcription of the token recurrence (a per-token Python loop
with numpy vector operations) used to cross-check ``gdn_oracle.c``; it shares
no code with the C oracle or the HIP library.

Recurrence (gated delta rule problem statement; decay applied before the
delta update, the order of the chunk recurrence on the state_summary.py
coverage page):

    h <- Diag(b^{g_t}) h
    h <- h + beta_t k_t (v_t - h^T k_t)^T
    o_t = scale * h^T q_t
"""
from __future__ import annotations

import numpy as np


def _decay(g, use_exp2):
    g = np.asarray(g, dtype=np.float64)
    return np.exp2(g) if use_exp2 else np.exp(g)


def fwd(q, k, v, g, beta, offsets, scale, *, gate_per_key=False, use_exp2=False, S0=None):
    """q, k: [N, H, K]; v: [N, H, V]; g: [N, H] or [N, H, K]; beta: [N, H].

    Returns (o [N, H, V], final [n_units, H, K, V]) in fp64."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); beta = np.asarray(beta, np.float64)
    N, H, K = k.shape
    V = v.shape[2]
    n_units = len(offsets) - 1
    o = np.zeros((N, H, V))
    final = np.zeros((n_units, H, K, V))
    for u in range(n_units):
        for hd in range(H):
            h = np.zeros((K, V)) if S0 is None else np.array(S0[u, hd], np.float64)
            for t in range(offsets[u], offsets[u + 1]):
                d = _decay(g[t, hd], use_exp2)
                h = (d[:, None] if gate_per_key else d) * h
                kt = k[t, hd]
                h = h + beta[t, hd] * np.outer(kt, v[t, hd] - kt @ h)
                o[t, hd] = scale * (q[t, hd] @ h)
            final[u, hd] = h
    return o, final


def summary(k, v, g, beta, offsets, *, gate_per_key=False, use_exp2=False):
    """Per-unit (S_ext [n_units, H, K, V], M [n_units, H, K, K])."""
    k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    N, H, K = k.shape
    V = v.shape[2]
    n_units = len(offsets) - 1
    S_ext = np.zeros((n_units, H, K, V))
    M = np.zeros((n_units, H, K, K))
    for u in range(n_units):
        for hd in range(H):
            s = np.zeros((K, V))
            m = np.eye(K)
            for t in range(offsets[u], offsets[u + 1]):
                d = _decay(g[t, hd], use_exp2)
                dd = d[:, None] if gate_per_key else d
                kt = k[t, hd]
                s = dd * s
                s = s + beta[t, hd] * np.outer(kt, v[t, hd] - kt @ s)
                m = dd * m
                m = m - beta[t, hd] * np.outer(kt, kt @ m)
            S_ext[u, hd] = s
            M[u, hd] = m
    return S_ext, M
