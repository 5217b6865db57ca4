"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes a value that the gated delta rule problem statement, the
pages' chunk/summary algebra or plain mathematics determines: a hand-derived
worked example, closed forms for degenerate inputs, invariants of the
recurrence, and an independent numpy transcription. A plausible slip in the
oracle (a dropped decay, a sign, an index off by one, a transposed state or
transfer map, the decay applied after instead of before the update) fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import twin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_2x2_worked.json")
# the oracle reads fp32 inputs: 0.6 and 0.8 in the worked example round at
# about 1e-8, so the hand values hold to about 1e-7
GOLDEN_TOL = 1e-6


def _rand(seed, N, H, K, V, per_key=False, gscale=0.1):
    r = np.random.default_rng(seed)
    q = r.standard_normal((N, H, K)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((N, H, K)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((N, H, V))
    g = -gscale * np.log1p(np.exp(r.standard_normal((N, H, K) if per_key else (N, H))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))
    f = lambda x: x.astype(np.float32)
    return f(q), f(k), f(v), f(g), f(beta)


# ---------------------------------------------------------------- worked example
@pytest.mark.parametrize("per_key", [False, True])
def test_golden_worked_example(per_key):
    gd = json.load(open(GOLDEN))
    k = np.array(gd["k"])[:, None, :]
    v = np.array(gd["v"])[:, None, :]
    q = np.array(gd["q"])[:, None, :]
    beta = np.array(gd["beta"])[:, None]
    g = np.array(gd["g_per_key"])[:, None, :] if per_key else np.array(gd["g_scalar"])[:, None]
    r = oracle.fwd(q, k, v, g, beta, [0, 3], gd["scale"], gate_per_key=per_key, use_exp2=True)
    tag = "per_key" if per_key else "scalar"
    np.testing.assert_allclose(r["o"][:, 0], gd["zero_start"]["o_" + tag], atol=GOLDEN_TOL)
    np.testing.assert_allclose(r["final"][0, 0], gd["zero_start"]["final_" + tag], atol=GOLDEN_TOL)
    if per_key:
        # the decay-after-update order is excluded by this example
        assert np.abs(r["final"][0, 0] - np.array(gd["decay_after_update_would_give_final_per_key"])).max() > 0.5


def test_golden_summary_and_start_state():
    gd = json.load(open(GOLDEN))
    k = np.array(gd["k"])[:, None, :]; v = np.array(gd["v"])[:, None, :]
    q = np.array(gd["q"])[:, None, :]; beta = np.array(gd["beta"])[:, None]
    g = np.array(gd["g_scalar"])[:, None]
    s = oracle.summary(k, v, g, beta, [0, 3], use_exp2=True)
    np.testing.assert_allclose(s["M"][0, 0], gd["zero_start"]["M_scalar"], atol=GOLDEN_TOL)
    np.testing.assert_allclose(s["S_ext"][0, 0], gd["zero_start"]["final_scalar"], atol=GOLDEN_TOL)
    S0 = np.array(gd["S0"])[None, None]
    r = oracle.fwd(q, k, v, g, beta, [0, 3], 1.0, use_exp2=True, S0=S0)
    np.testing.assert_allclose(r["o"][:, 0], gd["from_S0"]["o_scalar"], atol=GOLDEN_TOL)
    np.testing.assert_allclose(r["final"][0, 0], gd["from_S0"]["final_scalar"], atol=GOLDEN_TOL)


# ---------------------------------------------------------------- closed forms
def test_beta_zero_zero_state_gives_zero():
    q, k, v, g, beta = _rand(1, 200, 2, 16, 8)
    r = oracle.fwd(q, k, v, g, np.zeros_like(beta), [0, 200], 0.3)
    assert np.all(r["o"] == 0.0) and np.all(r["final"] == 0.0)


@pytest.mark.parametrize("per_key", [False, True])
def test_constant_state_decays_by_cumulative_gate(per_key):
    # beta = 0: h_t = Diag(b^{sum_{s<=t} g_s}) S0, o_t = scale h_t^T q_t
    N, H, K, V = 50, 2, 8, 6
    q, k, v, g, _ = _rand(2, N, H, K, V, per_key=per_key)
    S0 = np.random.default_rng(3).standard_normal((1, H, K, V))
    r = oracle.fwd(q, k, v, g, np.zeros((N, H), np.float32), [0, N], 0.7,
                   gate_per_key=per_key, S0=S0)
    G = np.cumsum(g.astype(np.float64), axis=0)
    for t in (0, 1, 17, N - 1):
        for hd in range(H):
            d = np.exp(G[t, hd])
            h = (d[:, None] if per_key else d) * S0[0, hd]
            np.testing.assert_allclose(r["o"][t, hd], 0.7 * q[t, hd].astype(np.float64) @ h,
                                       rtol=1e-12, atol=1e-14)


def test_single_token_closed_form():
    q, k, v, g, beta = _rand(4, 1, 3, 8, 5)
    r = oracle.fwd(q, k, v, g, beta, [0, 1], 0.25)
    for hd in range(3):
        qk = q[0, hd].astype(np.float64) @ k[0, hd].astype(np.float64)
        np.testing.assert_allclose(r["o"][0, hd], 0.25 * beta[0, hd] * qk * v[0, hd], rtol=1e-12)


def test_total_forgetting():
    # g = -1e4 (ln units): b^g = 0, so each token sees only its own write
    N, H, K, V = 40, 2, 8, 4
    q, k, v, _, beta = _rand(5, N, H, K, V)
    g = np.full((N, H), -1e4, np.float32)
    r = oracle.fwd(q, k, v, g, beta, [0, N], 1.0)
    qk = np.einsum("nhk,nhk->nh", q.astype(np.float64), k.astype(np.float64))
    np.testing.assert_allclose(r["o"], (beta * qk)[..., None] * v, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("per_key", [False, True])
def test_just_written_key_returns_its_value(per_key):
    # beta = 1 and a unit key: the update replaces the key's read-out, so
    # h_t^T k_t = v_t whatever the gate; reading with q_t = k_t returns scale * v_t.
    # With the decay applied after the update this fails for per-key gates.
    N, H, K, V = 64, 2, 16, 8
    _, k, v, g, _ = _rand(6, N, H, K, V, per_key=per_key, gscale=0.5)
    k64 = k.astype(np.float64)
    k = (k64 / np.linalg.norm(k64, axis=-1, keepdims=True)).astype(np.float32)
    r = oracle.fwd(k, k, v, g, np.ones((N, H), np.float32), [0, N], 0.5, gate_per_key=per_key)
    nk = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True) ** 2
    # exact up to the fp32 rounding of the unit keys (|k|^2 = 1 + O(1e-7))
    np.testing.assert_allclose(r["o"], 0.5 * v, atol=2e-6 * np.abs(v).max())
    assert nk.max() < 1 + 1e-6


def test_basis_key_retrieval_and_overwrite():
    # g = 0, beta = 1, keys are standard basis vectors: the state is a table of
    # the last value written to each key; querying e_i reads it (scale = 2^-3).
    rng = np.random.default_rng(7)
    N, K, V = 48, 8, 4
    widx = rng.integers(0, K, N)
    qidx = rng.integers(0, K, N)
    k = np.eye(K, dtype=np.float32)[widx][:, None]
    q = np.eye(K, dtype=np.float32)[qidx][:, None]
    v = rng.integers(-8, 9, (N, 1, V)).astype(np.float32)
    r = oracle.fwd(q, k, v, np.zeros((N, 1), np.float32), np.ones((N, 1), np.float32),
                   [0, N], 0.125)
    table = np.zeros((K, V))
    for t in range(N):
        table[widx[t]] = v[t, 0]
        assert np.array_equal(r["o"][t, 0], 0.125 * table[qidx[t]])


def test_orthonormal_keys_retrieve_values():
    # the spec check: g = 0, beta = 1, orthonormal keys: a key written
    # once is read back exactly (up to the keys' fp32 rounding)
    rng = np.random.default_rng(8)
    K = V = 16
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm.T.astype(np.float32)[:, None]          # K tokens, one key each
    v = rng.standard_normal((K, 1, V)).astype(np.float32)
    zeros = np.zeros((K, 1), np.float32)
    r = oracle.fwd(k, k, v, zeros, np.ones((K, 1), np.float32), [0, K], 1.0)
    S = r["final"][0, 0]
    for i in range(K):
        np.testing.assert_allclose(k[i, 0].astype(np.float64) @ S, v[i, 0], atol=1e-5)


# ---------------------------------------------------------------- invariants
def test_linear_in_values_and_start_state():
    N, H, K, V = 70, 2, 8, 6
    q, k, v1, g, beta = _rand(9, N, H, K, V)
    v2 = np.random.default_rng(10).standard_normal((N, H, V)).astype(np.float32)
    rng = np.random.default_rng(11)
    A = rng.standard_normal((1, H, K, V)); B = rng.standard_normal((1, H, K, V))
    r1 = oracle.fwd(q, k, v1, g, beta, [0, N], 1.0, S0=A)
    r2 = oracle.fwd(q, k, v2, g, beta, [0, N], 1.0, S0=B)
    # v1 + v2 rounds when stored in fp32 (relative 6e-8), hence the tolerance
    v12f = (v1.astype(np.float64) + v2.astype(np.float64)).astype(np.float32)
    r12 = oracle.fwd(q, k, v12f, g, beta, [0, N], 1.0, S0=A + B)
    np.testing.assert_allclose(r12["o"], r1["o"] + r2["o"], atol=1e-5 * np.abs(r12["o"]).max())
    np.testing.assert_allclose(r12["final"], r1["final"] + r2["final"], atol=1e-5 * np.abs(r12["final"]).max())


def test_heads_independent_and_permutable():
    N, H, K, V = 30, 4, 8, 4
    q, k, v, g, beta = _rand(12, N, H, K, V)
    perm = [2, 0, 3, 1]
    r = oracle.fwd(q, k, v, g, beta, [0, N], 0.5)
    rp = oracle.fwd(q[:, perm], k[:, perm], v[:, perm], g[:, perm], beta[:, perm], [0, N], 0.5)
    assert np.array_equal(rp["o"], r["o"][:, perm])
    rs = oracle.fwd(q, k, v, g, beta, [0, N], 0.5, heads=[3, 1])
    assert np.array_equal(rs["o"], r["o"][:, [3, 1]])


@pytest.mark.parametrize("per_key", [False, True])
def test_split_at_every_point_equals_unsplit(per_key):
    # end state = M S_entry + S_ext for any split point (state_summary.py
    # coverage page; the Sana distributed_scan.py page states the split scan
    # equals the scan of the concatenated sequence)
    N, H, K, V = 24, 1, 6, 5
    q, k, v, g, beta = _rand(13, N, H, K, V, per_key=per_key, gscale=0.02)
    S0 = np.random.default_rng(14).standard_normal((1, H, K, V))
    full = oracle.fwd(q, k, v, g, beta, [0, N], 1.0, gate_per_key=per_key, S0=S0)["final"][0]
    for s in range(0, N + 1):
        summ = oracle.summary(k, v, g, beta, [0, s, N], gate_per_key=per_key)
        S_init = oracle.merge(summ["S_ext"], summ["M"], S0[0])
        np.testing.assert_allclose(S_init[2], full, atol=1e-12)
        # the transposed transfer map does not reproduce it
        if 0 < s < N:
            Mt = np.swapaxes(summ["M"], -1, -2)
            wrong = oracle.merge(summ["S_ext"], Mt, S0[0])
            assert np.abs(wrong[2] - full).max() > 1e-3


def test_transfer_map_closed_forms():
    N, H, K, V = 20, 1, 6, 4
    q, k, v, g, beta = _rand(15, N, H, K, V, per_key=True)
    # beta = 0: M = Diag(b^{sum g})
    s = oracle.summary(k, v, g, np.zeros((N, H), np.float32), [0, N], gate_per_key=True)
    np.testing.assert_allclose(s["M"][0, 0], np.diag(np.exp(g.astype(np.float64).sum(0)[0])),
                               rtol=1e-12, atol=1e-15)
    assert np.all(s["S_ext"] == 0)
    # one token, g = 0, beta = 1, unit key: M = I - k k^T, a projector killing k
    kk = k[:1].astype(np.float64)
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    s1 = oracle.summary(kk.astype(np.float32), v[:1], np.zeros((1, 1, K), np.float32),
                        np.ones((1, 1), np.float32), [0, 1], gate_per_key=True)
    M = s1["M"][0, 0]
    np.testing.assert_allclose(M @ M, M, atol=1e-6)
    np.testing.assert_allclose(M @ kk[0, 0].astype(np.float32).astype(np.float64), 0, atol=1e-6)


def test_empty_segment_is_identity():
    q, k, v, g, beta = _rand(16, 10, 1, 4, 3)
    s = oracle.summary(k, v, g, beta, [0, 0, 10])
    assert np.array_equal(s["M"][0, 0], np.eye(4)) and np.all(s["S_ext"][0] == 0)


def test_packed_equals_separate_documents():
    N, H, K, V = 90, 2, 8, 4
    q, k, v, g, beta = _rand(17, N, H, K, V)
    cu = [0, 13, 64, 65, 90]
    packed = oracle.fwd(q, k, v, g, beta, cu, 0.3)
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        sep = oracle.fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a], 0.3)
        assert np.array_equal(packed["o"][a:b], sep["o"])
        assert np.array_equal(packed["final"][i], sep["final"][0])


def test_chunk_states_are_prefix_final_states():
    N, H, K, V = 150, 2, 8, 4
    q, k, v, g, beta = _rand(18, N, H, K, V)
    S0 = np.random.default_rng(19).standard_normal((1, H, K, V))
    r = oracle.fwd(q, k, v, g, beta, [0, N], 1.0, S0=S0, chunk_states=True, chunk=64)
    assert r["chunk_states"].shape[0] == 3
    assert np.array_equal(r["chunk_states"][0], S0[0])
    for c in (1, 2):
        pre = oracle.fwd(q[:64 * c], k[:64 * c], v[:64 * c], g[:64 * c], beta[:64 * c],
                         [0, 64 * c], 1.0, S0=S0)
        assert np.array_equal(r["chunk_states"][c], pre["final"][0])


def test_resume_equals_one_run():
    N, H, K, V = 100, 2, 8, 4
    q, k, v, g, beta = _rand(20, N, H, K, V)
    one = oracle.fwd(q, k, v, g, beta, [0, N], 1.0)
    a = oracle.fwd(q[:37], k[:37], v[:37], g[:37], beta[:37], [0, 37], 1.0)
    b = oracle.fwd(q[37:], k[37:], v[37:], g[37:], beta[37:], [0, N - 37], 1.0, S0=a["final"])
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]]), one["o"], atol=1e-13)
    np.testing.assert_allclose(b["final"], one["final"], atol=1e-13)


def test_per_key_uniform_gate_equals_scalar_gate():
    # a per-key log2 gate that is the same on every key equals the scalar ln gate
    N, H, K, V = 40, 2, 8, 4
    q, k, v, g, beta = _rand(21, N, H, K, V)
    g2 = (g.astype(np.float64) / math.log(2.0))
    g2f = g2.astype(np.float32)
    gln = (g2f.astype(np.float64) * math.log(2.0)).astype(np.float32)
    a = oracle.fwd(q, k, v, gln, beta, [0, N], 1.0)
    b = oracle.fwd(q, k, v, np.repeat(g2f[..., None], K, -1), beta, [0, N], 1.0,
                   gate_per_key=True, use_exp2=True)
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-6)


# ---------------------------------------------------------------- twin cross-check
@pytest.mark.parametrize("per_key,use_exp2", [(False, False), (True, True), (True, False)])
def test_c_oracle_matches_numpy_twin(per_key, use_exp2):
    N, H, K, V = 70, 2, 8, 6
    q, k, v, g, beta = _rand(22, N, H, K, V, per_key=per_key)
    cu = [0, 30, 70]
    S0 = np.random.default_rng(23).standard_normal((2, H, K, V))
    c = oracle.fwd(q, k, v, g, beta, cu, 0.4, gate_per_key=per_key, use_exp2=use_exp2, S0=S0)
    o, fin = twin.fwd(q, k, v, g, beta, cu, 0.4, gate_per_key=per_key, use_exp2=use_exp2, S0=S0)
    np.testing.assert_allclose(c["o"], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c["final"], fin, rtol=1e-12, atol=1e-13)
    cs = oracle.summary(k, v, g, beta, cu, gate_per_key=per_key, use_exp2=use_exp2)
    ext, M = twin.summary(k, v, g, beta, cu, gate_per_key=per_key, use_exp2=use_exp2)
    np.testing.assert_allclose(cs["S_ext"], ext, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cs["M"], M, rtol=1e-12, atol=1e-13)


def test_oracle_rejects_bad_offsets():
    q, k, v, g, beta = _rand(24, 10, 1, 4, 3)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, g, beta, [0, 6, 5, 10], 1.0)


@pytest.mark.parametrize("per_key,with_s0", [(False, False), (True, True), (False, True)])
def test_piece_merge_equals_prefix_states(per_key, with_s0):
    # every piece of a split packed sequence enters with the state that the
    # plain recurrence reaches at the piece's first token from its document's
    # start (first_state / last_state of the Diff Coverage page's packed plan)
    from oracle import varlen
    N, H, K, V = 40, 2, 5, 4
    q, k, v, g, beta = _rand(31, N, H, K, V, per_key=per_key, gscale=0.05)
    docs, segs = [0, 7, 26, 40], [0, 10, 13, 20, 33, 40]
    pieces, pdoc, _ = varlen.split_pieces(docs, segs)
    S0 = np.random.default_rng(32).standard_normal((len(docs) - 1, H, K, V)) if with_s0 else None
    summ = oracle.summary(k, v, g, beta, pieces, gate_per_key=per_key)
    S_in = oracle.merge_pieces(summ["S_ext"], summ["M"], pdoc, S0)
    for p, start in enumerate(pieces[:-1]):
        d = pdoc[p]
        if start == docs[d]:
            want = np.zeros((H, K, V)) if S0 is None else S0[d]
        else:
            want = oracle.fwd(q[docs[d]:start], k[docs[d]:start], v[docs[d]:start], g[docs[d]:start],
                              beta[docs[d]:start], [0, start - docs[d]], 1.0, gate_per_key=per_key,
                              S0=None if S0 is None else S0[d][None])["final"][0]
        np.testing.assert_allclose(S_in[p], want, atol=1e-12)
    # the correction forward over the pieces reproduces the packed forward
    whole = oracle.fwd(q, k, v, g, beta, docs, 0.7, gate_per_key=per_key, S0=S0)
    corr = oracle.fwd(q, k, v, g, beta, pieces, 0.7, gate_per_key=per_key, S0=S_in)
    np.testing.assert_allclose(corr["o"], whole["o"], atol=1e-12)
    last = [p for p in range(len(pdoc)) if p == len(pdoc) - 1 or pdoc[p + 1] != pdoc[p]]
    np.testing.assert_allclose(corr["final"][last], whole["final"], atol=1e-12)
    # carrying a state across a document boundary is wrong
    wrong = oracle.merge_pieces(summ["S_ext"], summ["M"], [0] * len(pdoc), S0 if S0 is None else S0[:1])
    assert np.abs(wrong - S_in).max() > 1e-3


# ---------------------------------------------------------------- v_new and the input transforms
@pytest.mark.parametrize("per_key", [False, True])
def test_v_new_rebuilds_the_chunk_state(per_key):
    # the chunk form h_L = Diag(b^{G_L}) h_0 + sum_j (k_j * b^{G_L - G_j}) v_new_j^T
    # (the state update of kda_split_state_summary_kernel on the state_summary.py
    # page) must hold with the oracle's per-token v_new, for any chunk length
    N, H, K, V = 23, 1, 5, 4
    q, k, v, g, beta = _rand(41, N, H, K, V, per_key=per_key, gscale=0.3)
    S0 = np.random.default_rng(42).standard_normal((1, H, K, V))
    r = oracle.fwd(q, k, v, g, beta, [0, N], 1.0, gate_per_key=per_key, S0=S0, want_v_new=True)
    gg = g.astype(np.float64)[:, 0]
    G = np.cumsum(gg, axis=0)
    GL = G[-1]
    dec = lambda x: np.exp(x)
    h = (dec(GL)[:, None] if per_key else dec(GL)) * S0[0, 0]
    for j in range(N):
        kj = k[j, 0].astype(np.float64) * (dec(GL - G[j]) if per_key else dec(GL - G[j]))
        h = h + np.outer(kj, r["v_new"][j, 0])
    np.testing.assert_allclose(h, r["final"][0, 0], atol=1e-12)
    # first token from a zero state writes beta_0 v_0; beta = 0 writes nothing
    z = oracle.fwd(q, k, v, g, beta, [0, N], 1.0, gate_per_key=per_key, want_v_new=True)
    np.testing.assert_allclose(z["v_new"][0, 0], float(beta[0, 0]) * v[0, 0].astype(np.float64), rtol=1e-14)
    b0 = oracle.fwd(q, k, v, g, np.zeros_like(beta), [0, N], 1.0, gate_per_key=per_key, want_v_new=True)
    assert np.all(b0["v_new"] == 0.0)


def test_qk_l2norm_is_scale_invariant():
    # the normalised forward does not see the scale of q and k; the raw one does
    N, H, K, V = 17, 2, 6, 3
    q, k, v, g, beta = _rand(43, N, H, K, V)
    rq = np.random.default_rng(44)
    # rows of different norms, all large enough that the epsilon (1e-6 under
    # the square root) moves nothing by more than about 1e-7
    q = (q * rq.uniform(2.0, 5.0, (N, H, 1))).astype(np.float32)
    k = (k * rq.uniform(2.0, 5.0, (N, H, 1))).astype(np.float32)
    a = oracle.fwd(q, k, v, g, beta, [0, 9, N], 0.7, qk_l2norm=True, want_v_new=True)
    b = oracle.fwd(3 * q, 2 * k, v, g, beta, [0, 9, N], 0.7, qk_l2norm=True, want_v_new=True)
    for key in ("o", "final", "v_new"):
        np.testing.assert_allclose(b[key], a[key], rtol=2e-6, atol=1e-7)
    raw = oracle.fwd(3 * q, 2 * k, v, g, beta, [0, 9, N], 0.7)
    assert np.abs(raw["o"] - a["o"]).max() > 1e-2
    # unit-norm inputs are left as they are (up to the epsilon in the norm)
    u = oracle.input_transforms(q, k, beta)
    qn, kn = u["q_hat"].astype(np.float32), u["k_hat"].astype(np.float32)
    c = oracle.fwd(qn, kn, v, g, beta, [0, 9, N], 0.7, qk_l2norm=True)
    d = oracle.fwd(qn, kn, v, g, beta, [0, 9, N], 0.7)
    np.testing.assert_allclose(c["o"], d["o"], rtol=1e-5, atol=1e-6)
    # what the slots hold: unit rows, and r = 1 / |x| up to the epsilon
    np.testing.assert_allclose(np.linalg.norm(u["q_hat"], axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(u["k_rstd"] * np.linalg.norm(k.astype(np.float64), axis=-1), 1.0, atol=1e-6)


def test_beta_sigmoid_closed_forms():
    N, H, K, V = 12, 1, 4, 4
    q, k, v, g, beta = _rand(45, N, H, K, V)
    zero = np.zeros_like(beta)
    half = np.full_like(beta, 0.5)
    a = oracle.fwd(q, k, v, g, zero, [0, N], 1.0, beta_sigmoid=True)
    b = oracle.fwd(q, k, v, g, half, [0, N], 1.0)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["final"], b["final"])   # sigmoid(0) = 1/2
    c = oracle.fwd(q, k, v, g, np.full_like(beta, -60.0), [0, N], 1.0, beta_sigmoid=True)
    d = oracle.fwd(q, k, v, g, zero, [0, N], 1.0)
    np.testing.assert_allclose(c["o"], d["o"], atol=1e-20)                                  # sigmoid(-60) ~ 1e-26
    x = np.linspace(-5, 5, 11)
    t = oracle.input_transforms(np.ones((11, 1, 2)), np.ones((11, 1, 2)), x)["beta_eff"]
    np.testing.assert_allclose(t + t[::-1], 1.0, atol=1e-15)                                 # sigmoid(x) + sigmoid(-x) = 1


@pytest.mark.parametrize("per_key", [False, True])
def test_split_identity_with_transforms(per_key):
    # S_end = M S_entry + S_ext holds for the transformed inputs too
    N, H, K, V = 20, 1, 5, 4
    q, k, v, g, beta = _rand(47, N, H, K, V, per_key=per_key, gscale=0.05)
    k = (k * 2.5).astype(np.float32)
    beta = (beta * 4 - 2).astype(np.float32)        # raw logits
    S0 = np.random.default_rng(48).standard_normal((1, H, K, V))
    kw = dict(gate_per_key=per_key, qk_l2norm=True, beta_sigmoid=True)
    full = oracle.fwd(q, k, v, g, beta, [0, N], 1.0, S0=S0, **kw)["final"][0]
    summ = oracle.summary(k, v, g, beta, [0, 7, N], **kw)
    S_init = oracle.merge(summ["S_ext"], summ["M"], S0[0])
    np.testing.assert_allclose(S_init[2], full, atol=1e-12)
