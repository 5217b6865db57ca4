"""Pins of the fp64 backward oracle (oracle.bwd), CPU only.

Nothing here reuses the backward's own formulas: every check compares it with
something fixed independently - central finite differences of the separate
numpy forward (oracle/twin.py, fp64 throughout), closed forms of one token, of
beta = 0 and of total forgetting, the adjoint of the affine segment summary
(dL/dS_start = M^T dL/dS_end + the segment's own contribution, the adjoint
merge of apply_kda_state_gradient_summary on the hyper-parallel Diff
Coverage page), and composition across a split point."""
import math

import numpy as np
import pytest

import oracle
from oracle import twin


def rng_inputs(seed, N, H, K, V, per_key, unit_norm=False, gate_scale=0.3):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    q, k, v = f(N, H, K), f(N, H, K), f(N, H, V)
    if unit_norm:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = (-gate_scale * np.log1p(np.exp(r.standard_normal((N, H, K) if per_key else (N, H))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((N, H))))).astype(np.float32)
    return q, k, v, g, beta


def loss(o, fin, do, dht):
    return float((o * do).sum() + (0.0 if dht is None else (fin * dht).sum()))


@pytest.mark.parametrize("per_key,use_exp2", [(False, False), (False, True), (True, True), (True, False)])
def test_backward_matches_finite_differences_of_the_twin(per_key, use_exp2):
    # two ragged units, two heads, K=4, V=3; an entry state and dL/dh_final
    N, H, K, V = 11, 2, 4, 3
    offs = [0, 5, 11]
    q, k, v, g, beta = rng_inputs(1 + per_key + 2 * use_exp2, N, H, K, V, per_key)
    r = np.random.default_rng(9)
    S0 = r.standard_normal((2, H, K, V))
    do = r.standard_normal((N, H, V))
    dht = r.standard_normal((2, H, K, V))
    scale = 0.7
    b = oracle.bwd(q, k, v, g, beta, offs, scale, do, gate_per_key=per_key, use_exp2=use_exp2, S0=S0, dht=dht)
    x = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64),
         "g": g.astype(np.float64), "beta": beta.astype(np.float64), "S0": S0.copy()}

    def L(xx):
        o, fin = twin.fwd(xx["q"], xx["k"], xx["v"], xx["g"], xx["beta"], offs, scale, gate_per_key=per_key,
                          use_exp2=use_exp2, S0=xx["S0"])
        return loss(o, fin, do, dht)

    eps = 1e-6
    for name, grad in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("S0", "dS0")):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (L(xp) - L(xm)) / (2 * eps)
        err = np.abs(fd - b[grad]).max() / max(1.0, np.abs(fd).max())
        assert err < 1e-7, f"{grad}: finite-difference mismatch {err:.2e}"


def test_one_token_closed_form():
    # T = 1 from an entry state S0, with d = e^g and the decayed state D = d S0:
    #   h_1 = D + b k (v - D^T k)^T,  o = scale h_1^T q,  L = o . do
    # so with u = v - D^T k and w = q - b (q.k) k:
    #   dq = scale h_1 do          dv = scale b (q.k) do
    #   dbeta = scale (q.k)(u.do)  dk = scale b [(u.do) q - (q.k) D do]
    #   dg = d scale w^T S0 do     dS0 = d scale w do^T
    K, V, scale = 5, 4, 0.5
    q, k, v, g, beta = rng_inputs(3, 1, 1, K, V, False)
    r = np.random.default_rng(4)
    S0 = r.standard_normal((1, 1, K, V))
    do = r.standard_normal((1, 1, V))
    b = oracle.bwd(q, k, v, g, beta, [0, 1], scale, do, S0=S0)
    qq, kk, vv, dd = (x[0, 0].astype(np.float64) for x in (q, k, v, do))
    bt, S = float(beta[0, 0]), S0[0, 0]
    d = math.exp(float(g[0, 0]))
    D = d * S
    h1 = D + bt * np.outer(kk, vv - D.T @ kk)
    u = vv - D.T @ kk
    w = qq - bt * (qq @ kk) * kk
    np.testing.assert_allclose(b["dq"][0, 0], scale * h1 @ dd, atol=1e-12)
    np.testing.assert_allclose(b["dv"][0, 0], scale * bt * (qq @ kk) * dd, atol=1e-12)
    np.testing.assert_allclose(b["dbeta"][0, 0], scale * (qq @ kk) * (u @ dd), atol=1e-12)
    np.testing.assert_allclose(b["dk"][0, 0], scale * bt * ((u @ dd) * qq - (qq @ kk) * (D @ dd)), atol=1e-12)
    np.testing.assert_allclose(b["dg"][0, 0], d * scale * (w @ S @ dd), atol=1e-12)
    np.testing.assert_allclose(b["dS0"][0, 0], d * scale * np.outer(w, dd), atol=1e-12)


def test_beta_zero_closed_form():
    # beta = 0 and S0 = 0 keep h = 0: dq, dk, dv and dg are zero,
    # dbeta_t = scale sum_{t' >= t} b^{G_t' - G_t} (q_t' . k_t)(do_t' . v_t)
    # and dS0 = scale sum_t b^{G_t} q_t do_t^T (G the inclusive cumulative gate)
    N, H, K, V, scale = 9, 2, 4, 3, 0.8
    q, k, v, g, beta = rng_inputs(5, N, H, K, V, False)
    beta[:] = 0
    do = np.random.default_rng(6).standard_normal((N, H, V))
    b = oracle.bwd(q, k, v, g, beta, [0, N], scale, do)
    for name in ("dq", "dk", "dv", "dg"):
        assert np.abs(b[name]).max() == 0.0, name
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    G = np.cumsum(g.astype(np.float64), axis=0)
    dS0 = scale * np.einsum("th,thk,thv->hkv", np.exp(G), q.astype(np.float64), do)
    np.testing.assert_allclose(b["dS0"][0], dS0, rtol=1e-12, atol=1e-14)
    ref = np.zeros((N, H))
    for t in range(N):
        for tp in range(t, N):
            ref[t] += scale * np.exp(G[tp] - G[t]) * np.einsum("hk,hk->h", q64[tp], k64[t]) * \
                np.einsum("hv,hv->h", do[tp], v64[t])
    np.testing.assert_allclose(b["dbeta"], ref, rtol=1e-12, atol=1e-14)


def test_total_forgetting_closed_form():
    # g = -1e4: each token sees only its own write, o_t = scale b_t (q_t.k_t) v_t
    N, H, K, V, scale = 7, 2, 4, 3, 0.6
    q, k, v, g, beta = rng_inputs(7, N, H, K, V, False)
    g[:] = -1e4
    do = np.random.default_rng(8).standard_normal((N, H, V))
    b = oracle.bwd(q, k, v, g, beta, [0, N], scale, do)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    qk = np.einsum("thk,thk->th", q, k)
    vd = np.einsum("thv,thv->th", v, do)
    bt = beta.astype(np.float64)
    np.testing.assert_allclose(b["dq"], scale * (bt * vd)[..., None] * k, atol=1e-12)
    np.testing.assert_allclose(b["dk"], scale * (bt * vd)[..., None] * q, atol=1e-12)
    np.testing.assert_allclose(b["dv"], scale * (bt * qk)[..., None] * do, atol=1e-12)
    np.testing.assert_allclose(b["dbeta"], scale * qk * vd, atol=1e-12)
    assert np.abs(b["dg"]).max() == 0.0 and np.abs(b["dS0"]).max() == 0.0


@pytest.mark.parametrize("per_key", [False, True])
def test_adjoint_of_the_segment_summary(per_key):
    # a segment maps S_start to M S_start + S_ext (oracle.summary), so
    # dL/dS_start = M^T dL/dS_end + (dL/dS_start with dL/dS_end = 0)
    N, H, K, V = 70, 2, 5, 4
    offs = [0, 30, 70]
    q, k, v, g, beta = rng_inputs(11, N, H, K, V, per_key, unit_norm=True, gate_scale=0.02)
    r = np.random.default_rng(12)
    S0 = r.standard_normal((2, H, K, V))
    do = r.standard_normal((N, H, V))
    dht = r.standard_normal((2, H, K, V))
    kw = dict(gate_per_key=per_key, use_exp2=per_key, S0=S0)
    full = oracle.bwd(q, k, v, g, beta, offs, 0.4, do, dht=dht, **kw)
    local = oracle.bwd(q, k, v, g, beta, offs, 0.4, do, **kw)
    M = oracle.summary(k, v, g, beta, offs, gate_per_key=per_key, use_exp2=per_key)["M"]
    assert np.abs(M - np.eye(K)).max() > 0.05                      # far from trivial
    ref = np.einsum("uhij,uhiv->uhjv", M, dht) + local["dS0"]
    np.testing.assert_allclose(full["dS0"], ref, rtol=1e-10, atol=1e-12)
    # a transposed transfer map does not satisfy it
    wrong = np.einsum("uhij,uhjv->uhiv", M, dht) + local["dS0"]
    assert np.abs(wrong - full["dS0"]).max() > 1e-3


def test_backward_composes_across_a_split():
    # one unit of 150 tokens == its halves [0, 70) and [70, 150), the second
    # run from the first half's end state, the first given the second's dL/dS0
    N, H, K, V, scale = 150, 1, 4, 4, 0.5
    q, k, v, g, beta = rng_inputs(13, N, H, K, V, False, gate_scale=0.05)
    r = np.random.default_rng(14)
    do = r.standard_normal((N, H, V))
    dht = r.standard_normal((1, H, K, V))
    full = oracle.bwd(q, k, v, g, beta, [0, N], scale, do, dht=dht)
    mid = oracle.fwd(q[:70], k[:70], v[:70], g[:70], beta[:70], [0, 70], scale)["final"]
    sl = lambda a, lo, hi: np.ascontiguousarray(a[lo:hi])
    second = oracle.bwd(*(sl(a, 70, N) for a in (q, k, v, g, beta)), [0, 80], scale, do[70:], S0=mid, dht=dht)
    first = oracle.bwd(*(sl(a, 0, 70) for a in (q, k, v, g, beta)), [0, 70], scale, do[:70], dht=second["dS0"])
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        np.testing.assert_allclose(np.concatenate([first[name], second[name]]), full[name], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(first["dS0"], full["dS0"], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("with_dht", [False, True])
def test_merge_adjoint_gives_the_unsplit_backward(with_dht):
    # one unit cut into four segments: local gradient summaries (each
    # segment's backward with a zero exit gradient, from its true entry
    # state), the reverse wavefront through oracle.merge_adjoint, then each
    # segment's backward from its exit gradient reproduce the unsplit
    # backward and dL/dS0
    N, H, K, V, scale = 130, 1, 4, 3, 0.6
    q, k, v, g, beta = rng_inputs(15, N, H, K, V, False, gate_scale=0.05)
    r = np.random.default_rng(16)
    do = r.standard_normal((N, H, V))
    S0 = r.standard_normal((1, H, K, V))
    dht = r.standard_normal((1, H, K, V)) if with_dht else None
    full = oracle.bwd(q, k, v, g, beta, [0, N], scale, do, S0=S0, dht=dht)
    cuts = [0, 20, 64, 65, N]
    S_in = oracle.merge(oracle.summary(k, v, g, beta, cuts)["S_ext"], oracle.summary(k, v, g, beta, cuts)["M"], S0[0])
    sl = lambda a, lo, hi: np.ascontiguousarray(a[lo:hi])
    seg = lambda s: [sl(a, cuts[s], cuts[s + 1]) for a in (q, k, v, g, beta)]
    local = [oracle.bwd(*seg(s), [0, cuts[s + 1] - cuts[s]], scale, do[cuts[s]:cuts[s + 1]],
                        S0=S_in[s][None])["dS0"][0] for s in range(4)]
    M = oracle.summary(k, v, g, beta, cuts)["M"]
    exits, G0 = oracle.merge_adjoint(np.stack(local), M, None if dht is None else dht[0])
    np.testing.assert_allclose(G0, full["dS0"][0], rtol=1e-10, atol=1e-12)
    parts = [oracle.bwd(*seg(s), [0, cuts[s + 1] - cuts[s]], scale, do[cuts[s]:cuts[s + 1]], S0=S_in[s][None],
                        dht=exits[s][None]) for s in range(4)]
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        np.testing.assert_allclose(np.concatenate([p[name] for p in parts]), full[name], rtol=1e-10, atol=1e-12)
    # the forward map (not its transpose) fails
    bad, _ = oracle.merge_adjoint(np.stack(local), np.swapaxes(M, -1, -2), None if dht is None else dht[0])
    wrong = oracle.bwd(*seg(0), [0, 20], scale, do[:20], S0=S_in[0][None], dht=bad[0][None])
    assert np.abs(wrong["dk"] - full["dk"][:20]).max() > 1e-4    # dq does not see the exit gradient
