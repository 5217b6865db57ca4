"""fp64 CPU oracle of the gated delta rule forward.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` are the only code allowed to import it. It shares
no code with the HIP library in ``chunked_gated_delta_05_amd``; the two meet
only in the seeded input generator, which holds none of the method's
arithmetic.

The C library ``gdn_oracle.c`` holds the arithmetic; this module loads it
with ctypes and converts numpy arrays. ``twin.py`` is an independent numpy
transcription used to cross-check it on tiny inputs; ``varlen.py`` defines the
packed-sequence chunk metadata.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [
            ctypes.c_int64, _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            _f64p, ctypes.c_int64, _i64p, _f64p, _f64p, ctypes.c_int64, _f64p,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, _f64p, ctypes.c_int]
        lib.gdn_oracle_summary.restype = ctypes.c_int
        lib.gdn_oracle_summary.argtypes = [
            ctypes.c_int64, _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, _i64p,
            _f64p, _f64p, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.gdn_oracle_merge.restype = ctypes.c_int
        lib.gdn_oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, _f64p, _f64p, _f64p, _f64p]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [
            ctypes.c_int64, _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def max_threads() -> int:
    return int(_lib().gdn_oracle_max_threads())


L2NORM_EPS = 1e-6   # the epsilon of the native prepare (Diff Coverage page)


def fwd(q, k, v, g, beta, offsets, scale, *, gate_per_key=False, use_exp2=False, S0=None,
        heads=None, want_o=True, want_final=True, chunk_states=False, chunk=64, qk_l2norm=False,
        beta_sigmoid=False, eps=L2NORM_EPS, want_v_new=False, threads=0):
    """Token-by-token forward in fp64.

    q, k: [N, H, K]; v: [N, H, V] (N = flat token count); g: [N, H] (scalar
    gate) or [N, H, K] (per-key gate); beta: [N, H]; offsets: unit token
    offsets (length n_units + 1); S0: [n_units, H, K, V] or None (zeros);
    heads: optional list of head indices to run (outputs are indexed by the
    position in that list).

    qk_l2norm / beta_sigmoid: the in-kernel input transforms (q and k
    L2-normalised with ``eps`` inside the square root, beta through a
    sigmoid) applied before the recurrence.

    Returns a dict with ``o`` [N, n_sel, V], ``final`` [n_units, n_sel, K, V],
    ``chunk_states`` [n_chunks, n_sel, K, V] (the state entering each
    ``chunk``-token block of every unit) and ``v_new`` [N, n_sel, V] (the
    value each token writes, beta_t (v_t - h~^T k_t)) as requested.
    """
    q, k, v, g, beta = _f32(q), _f32(k), _f32(v), _f32(g), _f32(beta)
    N, H, K = k.shape
    V = v.shape[2]
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n_units = len(offs) - 1
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    n_sel = H if sel is None else len(sel)
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    if s0 is not None and s0.shape != (n_units, H, K, V):
        raise ValueError("S0 must be [n_units, H, K, V]")
    o = np.zeros((N, n_sel, V)) if want_o else None
    fin = np.zeros((n_units, n_sel, K, V)) if want_final else None
    cs = None
    if chunk_states:
        n_chunks = int(sum((b - a + chunk - 1) // chunk for a, b in zip(offs[:-1], offs[1:])))
        cs = np.zeros((n_chunks, n_sel, K, V))
    vn = np.zeros((N, n_sel, V)) if want_v_new else None
    rc = _lib().gdn_oracle_fwd(
        n_units, _ptr(offs, _i64p), H, K, V, _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
        _ptr(g, _f32p), _ptr(beta, _f32p), int(gate_per_key), int(use_exp2), float(scale),
        _ptr(s0, _f64p), n_sel, _ptr(sel, _i64p), _ptr(o, _f64p), _ptr(fin, _f64p), int(chunk),
        _ptr(cs, _f64p), int(qk_l2norm), int(beta_sigmoid), float(eps), _ptr(vn, _f64p), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"o": o, "final": fin, "chunk_states": cs, "v_new": vn}


def summary(k, v, g, beta, offsets, *, gate_per_key=False, use_exp2=False, heads=None,
            want_ext=True, want_M=True, qk_l2norm=False, beta_sigmoid=False, eps=L2NORM_EPS, threads=0):
    """Per-unit segment summaries: S_ext [n_units, n_sel, K, V] (state reached
    from zero) and M [n_units, n_sel, K, K] (the map applied to an entry
    state), so that the state at the end of a unit is M @ S_entry + S_ext."""
    k, v, g, beta = _f32(k), _f32(v), _f32(g), _f32(beta)
    N, H, K = k.shape
    V = v.shape[2]
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n_units = len(offs) - 1
    sel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    n_sel = H if sel is None else len(sel)
    ext = np.zeros((n_units, n_sel, K, V)) if want_ext else None
    M = np.zeros((n_units, n_sel, K, K)) if want_M else None
    rc = _lib().gdn_oracle_summary(
        n_units, _ptr(offs, _i64p), H, K, V, _ptr(k, _f32p), _ptr(v, _f32p), _ptr(g, _f32p),
        _ptr(beta, _f32p), int(gate_per_key), int(use_exp2), n_sel, _ptr(sel, _i64p),
        _ptr(ext, _f64p), _ptr(M, _f64p), int(qk_l2norm), int(beta_sigmoid), float(eps), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"S_ext": ext, "M": M}


def merge(S_ext, M, S0=None):
    """S_ext: [n_seg, n, K, V]; M: [n_seg, n, K, K]; S0: [n, K, V] or None.

    Returns S_init [n_seg + 1, n, K, V]: the state entering every segment,
    then the state at the end of the last one."""
    ext = np.ascontiguousarray(np.asarray(S_ext, dtype=np.float64))
    m = np.ascontiguousarray(np.asarray(M, dtype=np.float64))
    n_seg, n, K, V = ext.shape
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    out = np.zeros((n_seg + 1, n, K, V))
    rc = _lib().gdn_oracle_merge(n_seg, n, K, V, _ptr(ext, _f64p), _ptr(m, _f64p),
                                 _ptr(s0, _f64p), _ptr(out, _f64p))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def merge_adjoint(dS_ext, M, dS_final=None):
    """Reverse wavefront of a split backward in fp64 (the adjoint summary of
    apply_kda_state_gradient_summary on the Diff Coverage page): with
    G_n = dS_final (zero when None) and G_s = M_s^T G_{s+1} + dS_ext[s],
    returns (dS_exit [n_seg, n, K, V] = G_{s+1} per segment, G_0).
    dS_ext: [n_seg, n, K, V]; M: [n_seg, n, K, K]; dS_final: [n, K, V]."""
    e = np.asarray(dS_ext, dtype=np.float64)
    m = np.asarray(M, dtype=np.float64)
    n_seg = e.shape[0]
    G = np.zeros(e.shape[1:]) if dS_final is None else np.asarray(dS_final, dtype=np.float64).copy()
    exits = np.zeros_like(e)
    for s in range(n_seg - 1, -1, -1):
        exits[s] = G
        G = np.swapaxes(m[s], -1, -2) @ G + e[s]
    return exits, G


def input_transforms(q, k, beta, eps=L2NORM_EPS):
    """The transformed inputs and their slots, in fp64: q_hat = q r_q and
    k_hat = k r_k with r = 1 / sqrt(sum x^2 + eps) per (token, head), and
    beta_eff = 1 / (1 + e^{-beta}) (use_qk_l2norm_in_kernel and
    use_beta_sigmoid_in_kernel of the native prepare, Diff Coverage page)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rq = 1.0 / np.sqrt((q * q).sum(-1) + eps)
    rk = 1.0 / np.sqrt((k * k).sum(-1) + eps)
    be = 1.0 / (1.0 + np.exp(-np.asarray(beta, dtype=np.float64)))
    return {"q_hat": q * rq[..., None], "k_hat": k * rk[..., None], "q_rstd": rq, "k_rstd": rk, "beta_eff": be}


def merge_pieces(S_ext, M, piece_doc, S0_docs=None):
    """Entry state of every piece of a split packed sequence, in fp64.

    S_ext: [n_pieces, n, K, V]; M: [n_pieces, n, K, K]; piece_doc: document of
    each piece (non-decreasing); S0_docs: [n_docs, n, K, V] or None.
    Follows first_state / last_state of PackedSequenceInfo on the Diff
    Coverage page: a piece that starts its document enters with that
    document's initial state (zero without one); a piece that continues its
    document enters with the previous piece's exit state, M S_in + S_ext, the
    affine summary rule of the state_summary.py page."""
    ext = np.asarray(S_ext, dtype=np.float64)
    m = np.asarray(M, dtype=np.float64)
    n_pieces, n, K, V = ext.shape
    out = np.zeros((n_pieces, n, K, V))
    for p in range(n_pieces):
        if p > 0 and piece_doc[p] == piece_doc[p - 1]:
            out[p] = m[p - 1] @ out[p - 1] + ext[p - 1]
        elif S0_docs is not None:
            out[p] = np.asarray(S0_docs, dtype=np.float64)[piece_doc[p]]
    return out


def bwd(q, k, v, g, beta, offsets, scale, dout, *, gate_per_key=False, use_exp2=False, S0=None,
        dht=None, threads=0):
    """Backward of ``fwd`` in fp64 (reverse mode of the token recurrence).

    dout: [N, H, V] (dL/do); dht: [n_units, H, K, V] (dL/dh_final) or None.
    Returns a dict of fp64 arrays: dq, dk [N, H, K], dv [N, H, V], dbeta
    [N, H], dg [N, H] (scalar gate) or [N, H, K] (per key) and dS0
    [n_units, H, K, V] (dL/dS0)."""
    q, k, v, g, beta = _f32(q), _f32(k), _f32(v), _f32(g), _f32(beta)
    N, H, K = k.shape
    V = v.shape[2]
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n_units = len(offs) - 1
    f64 = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    s0, do, dh = f64(S0), f64(dout), f64(dht)
    if do.shape != (N, H, V):
        raise ValueError("dout must be [N, H, V]")
    for a, shp in ((s0, (n_units, H, K, V)), (dh, (n_units, H, K, V))):
        if a is not None and a.shape != shp:
            raise ValueError("states must be [n_units, H, K, V]")
    out = {"dq": np.zeros((N, H, K)), "dk": np.zeros((N, H, K)), "dv": np.zeros((N, H, V)),
           "dbeta": np.zeros((N, H)), "dg": np.zeros((N, H, K) if gate_per_key else (N, H)),
           "dS0": np.zeros((n_units, H, K, V))}
    rc = _lib().gdn_oracle_bwd(
        n_units, _ptr(offs, _i64p), H, K, V, _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
        _ptr(g, _f32p), _ptr(beta, _f32p), int(gate_per_key), int(use_exp2), float(scale),
        _ptr(s0, _f64p), _ptr(do, _f64p), _ptr(dh, _f64p), _ptr(out["dq"], _f64p), _ptr(out["dk"], _f64p),
        _ptr(out["dv"], _f64p), _ptr(out["dg"], _f64p), _ptr(out["dbeta"], _f64p), _ptr(out["dS0"], _f64p),
        int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out
