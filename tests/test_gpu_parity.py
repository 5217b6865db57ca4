"""Parity of the HIP forward (through the C ABI) with the fp64 oracle.

Tolerances: max |x - oracle| <= tol * rms(oracle) with tol = 1e-4 for fp32
inputs and 2e-2 for bf16 inputs (fp32 accumulation, fp32 output o). Exact
cases (zero writes, basis-key tables) are compared bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_05_amd import binding as gb
from chunked_gated_delta_05_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, flat_inputs, np32, rel_err, unit_offsets

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(B=1, T=200, H=3, dtype="bf16", per_key=False, use_exp2=False, gate_coef=0.1,
          layout="BSND", n_docs=0, doc_len=(100, 4000), n_seg=0):
    return W.Workload("small", B=B, T=T, H=H, dtype=dtype, layout=layout, gate_per_key=per_key,
                      use_exp2=use_exp2, gate_coef=gate_coef, n_docs=n_docs, doc_len=doc_len,
                      n_seg=n_seg)


def to_dev(d):
    out = dict(d)
    for n in ("q", "k", "v", "g", "beta"):
        out[n] = d[n].to(DEV)
    return out


def run_gpu(d, meta=None, **kw):
    w = d["workload"]
    if meta is None and d["offsets"] is not None and w.layout == "TND":
        meta = gb.make_meta(d["offsets"], w.T, DEV)
    o, fin, ex = gb.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], meta=meta,
                                  use_exp2=w.use_exp2, **kw)
    torch.cuda.synchronize()
    return o, fin, ex


def run_oracle(d, offsets=None, heads=None, S0=None, **kw):
    q, k, v, g, beta = flat_inputs(d)
    w = d["workload"]
    return oracle.fwd(q, k, v, g, beta, offsets or unit_offsets(d), d["scale"],
                      gate_per_key=w.gate_per_key, use_exp2=w.use_exp2, heads=heads, S0=S0, **kw)


def flat_o(o, w):
    return np32(o.reshape(-1, *o.shape[2:]) if w.layout == "BSND" else o)


# ------------------------------------------------------------------ small shapes
@pytest.mark.parametrize("B,T,H", [(1, 64, 1), (2, 200, 3), (1, 1, 2), (1, 130, 2), (3, 63, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dense_small(B, T, H, dtype):
    print(f"dense B={B} T={T} H={H} {dtype}", flush=True)
    d = to_dev(W.generate(small(B=B, T=T, H=H, dtype=dtype), 11 + T))
    o, fin, ex = run_gpu(d, output_final_state=True, want_h=True, want_g_cumsum=True)
    r = run_oracle(d, chunk_states=True)
    w = d["workload"]
    tol = TOL[dtype]
    assert_close(flat_o(o, w), r["o"], tol, "o")
    assert_close(np32(fin), r["final"], tol, "final state")
    assert_close(np32(ex["h"]), r["chunk_states"], tol, "chunk entry states")
    gc = np32(ex["g_cumsum"]).reshape(B, T, H)
    ref = np.zeros((B, T, H))
    gg = np32(d["g"]).astype(np.float64)
    for c0 in range(0, T, 64):
        ref[:, c0:c0 + 64] = np.cumsum(gg[:, c0:c0 + 64], axis=1)
    np.testing.assert_allclose(gc, ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_scalar_gate_base2(dtype):
    # scalar gate in log2 units (decay 2^g), ragged tail, entry and final states
    print(f"scalar gate base 2 {dtype}", flush=True)
    w = small(B=2, T=150, H=3, dtype=dtype, use_exp2=True, gate_coef=0.05)
    d = to_dev(W.generate(w, 83))
    S0 = (torch.randn(2, 3, 128, 128, generator=torch.Generator().manual_seed(6)) * 0.3).to(DEV)
    o, fin, ex = run_gpu(d, initial_state=S0, output_final_state=True, want_h=True)
    r = run_oracle(d, S0=np32(S0).astype(np.float64), chunk_states=True)
    tol = TOL[dtype]
    assert_close(flat_o(o, w), r["o"], tol, "base-2 o")
    assert_close(np32(fin), r["final"], tol, "base-2 final")
    assert_close(np32(ex["h"]), r["chunk_states"], tol, "base-2 chunk states")


def test_many_heads():
    # 40 heads: head strides of 10 KiB per token row in q, k, v and o
    print("many heads", flush=True)
    w = small(B=1, T=130, H=40)
    d = to_dev(W.generate(w, 89))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    assert_close(flat_o(o, w), r["o"], TOL["bf16"], "40-head o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "40-head final")


@pytest.mark.parametrize("per_key", [False, True])
def test_bf16_output_is_the_rounded_fp32_output(per_key):
    # o_dtype = bf16 stores the same fp32 result rounded to nearest-even:
    # within half a bf16 ulp of the fp32-output run (allowing one ulp for
    # reassociation between the two instantiations)
    print(f"bf16 output per_key={per_key}", flush=True)
    d = to_dev(W.generate(small(B=2, T=200, H=3, per_key=per_key, use_exp2=per_key,
                                gate_coef=0.05 if per_key else 0.1), 29))
    o32, _, _ = run_gpu(d)
    o16, _, _ = run_gpu(d, o_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    ref = np32(o32).astype(np.float64)
    got = np32(o16).astype(np.float64)
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - ref) <= ulp), float(np.max(np.abs(got - ref) / ulp))


def test_tiny_fp32_workload():
    d = to_dev(W.generate(W.WORKLOADS[0], 1000))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    e = assert_close(flat_o(o, d["workload"]), r["o"], TOL["fp32"], "o")
    assert_close(np32(fin), r["final"], TOL["fp32"], "final")
    print(f"gdn_tiny_fp32 o err/rms {e:.2e}")


def test_initial_state_and_resume():
    d = to_dev(W.generate(small(B=2, T=256, H=2), 5))
    S0 = torch.randn(2, 2, 128, 128, device=DEV) * 0.3
    o, fin, _ = run_gpu(d, initial_state=S0, output_final_state=True)
    r = run_oracle(d, S0=np32(S0).astype(np.float64))
    assert_close(flat_o(o, d["workload"]), r["o"], TOL["bf16"], "o with S0")
    assert_close(np32(fin), r["final"], TOL["bf16"], "final with S0")
    # two calls over [0,128) and [128,256) with the state handed over
    half = {n: d[n][:, :128].contiguous() for n in ("q", "k", "v", "g", "beta")}
    rest = {n: d[n][:, 128:].contiguous() for n in ("q", "k", "v", "g", "beta")}
    for x in (half, rest):
        x.update(scale=d["scale"], offsets=None, workload=small(B=2, T=128, H=2))
    o1, f1, _ = run_gpu(half, initial_state=S0, output_final_state=True)
    o2, f2, _ = run_gpu(rest, initial_state=f1, output_final_state=True)
    np.testing.assert_allclose(np32(torch.cat([o1, o2], 1)), np32(o), rtol=0, atol=1e-4 * float(o.abs().max()))
    np.testing.assert_allclose(np32(f2), np32(fin), rtol=0, atol=1e-4 * float(fin.abs().max()))


def test_prep_slots_inverse_residual():
    # A slot: T = (I + L)^{-1}; check (I + L) T = I with L rebuilt in fp64
    d = to_dev(W.generate(small(B=1, T=150, H=2), 21))
    _, _, ex = run_gpu(d, want_A=True)
    A = np32(ex["A"]).astype(np.float64)            # [T, H, 64]
    k = np32(d["k"][0]).astype(np.float64)
    beta = np32(d["beta"][0]).astype(np.float64)
    g = np32(d["g"][0]).astype(np.float64)
    for h in range(2):
        for c0 in range(0, 150, 64):
            n = min(64, 150 - c0)
            G = np.cumsum(g[c0:c0 + n, h])
            kk = k[c0:c0 + n, h]
            L = np.tril(beta[c0:c0 + n, h, None] * (kk @ kk.T) * np.exp(G[:, None] - G[None, :]), -1)
            Tm = A[c0:c0 + n, h, :n]
            res = (np.eye(n) + L) @ Tm - np.eye(n)
            assert np.abs(res).max() < 1e-5, np.abs(res).max()


def test_prep_slots_per_key():
    # per-key gate (log2 units): g_cumsum against the fp64 per-key prefix sum,
    # (I + L) T = I with L_ij = beta_i sum_d k_id k_jd 2^{G_id - G_jd} rebuilt
    # in fp64, and the chunk entry states against the oracle
    T, H = 150, 2
    print(f"per-key slots T={T} H={H}", flush=True)
    d = to_dev(W.generate(small(B=1, T=T, H=H, per_key=True, use_exp2=True, gate_coef=0.05), 23))
    _, _, ex = run_gpu(d, want_A=True, want_g_cumsum=True, want_h=True)
    A = np32(ex["A"]).astype(np.float64)            # [T, H, 64]
    gc = np32(ex["g_cumsum"]).astype(np.float64)[0]  # [T, H, K]
    k = np32(d["k"][0]).astype(np.float64)
    beta = np32(d["beta"][0]).astype(np.float64)
    g = np32(d["g"][0]).astype(np.float64)
    for h in range(H):
        for c0 in range(0, T, 64):
            n = min(64, T - c0)
            G = np.cumsum(g[c0:c0 + n, h], axis=0)                     # [n, K]
            np.testing.assert_allclose(gc[c0:c0 + n, h], G, rtol=1e-5, atol=1e-5)
            kk = k[c0:c0 + n, h]
            D = np.exp2(G[:, None, :] - G[None, :, :])                  # [i, j, K]
            bt = beta[c0:c0 + n, h, None]
            L = np.tril(bt * np.einsum("id,jd,ijd->ij", kk, kk, D), -1)
            Tm = A[c0:c0 + n, h, :n]
            res = (np.eye(n) + L) @ Tm - np.eye(n)
            # the gated keys enter the L product as fp16 operands (two
            # roundings of 2^-11 relative each), so |L_gpu - L| <= 2.01 2^-11
            # L_abs elementwise and the residual (L - L_gpu) T is bounded by
            # that times |T|
            L_abs = np.tril(bt * np.einsum("id,jd,ijd->ij", np.abs(kk), np.abs(kk), D), -1)
            bound = 2.01 * 2.0 ** -11 * (L_abs @ np.abs(Tm)) + 1e-5
            assert (np.abs(res) <= bound).all(), float((np.abs(res) / bound).max())
    r = run_oracle(d, chunk_states=True)
    assert_close(np32(ex["h"]), r["chunk_states"], TOL["bf16"], "per-key chunk entry states")


# ------------------------------------------------------------------ exact cases
@pytest.mark.parametrize("layout", ["BSND", "TND"])
def test_marshalled_call_matches_forward(layout):
    # FwdCall (arguments marshalled once) and its two stages (prepare only,
    # then reuse) give the forward's output and final state bit for bit
    print(f"marshalled call {layout}", flush=True)
    if layout == "BSND":
        d = to_dev(W.generate(small(B=2, T=200, H=3), 41))
        meta = None
    else:
        cu = W.cu_from_lengths([30, 200, 64, 9])
        base = W.generate(small(B=1, T=cu[-1], H=3), 43)
        d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
        d.update(scale=base["scale"], offsets=cu,
                 workload=small(B=1, T=cu[-1], H=3, layout="TND", n_docs=4))
        meta = gb.make_meta(cu, cu[-1], DEV)
    o_ref, fin_ref, _ = run_gpu(d, meta=meta, output_final_state=True)
    ws = torch.empty(gb.workspace_bytes(gb._desc(d["k"], 3, d["k"].dtype, torch.float32, False, False,
                                                 d["scale"], meta)), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(o_ref)
    fin = torch.empty_like(fin_ref)
    call = gb.FwdCall(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], out=o, workspace=ws,
                      meta=meta, final_out=fin)
    call(0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(fin, fin_ref)
    o.zero_()
    fin.zero_()
    call(gb.FLAG_PREPARE_ONLY)
    call(gb.FLAG_REUSE_PREPARED)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(fin, fin_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_empty_sequence_returns_entry_state(dtype):
    # T = 0: no chunk to prepare, the state passes take zero steps, and the
    # final state is the entry state (or zero)
    print(f"empty sequence {dtype}", flush=True)
    d = to_dev(W.generate(small(B=2, T=0, H=3, dtype=dtype), 17))
    S0 = torch.randn(2, 3, 128, 128, generator=torch.Generator().manual_seed(9)).to(DEV)
    o, fin, _ = run_gpu(d, initial_state=S0, output_final_state=True)
    assert o.numel() == 0
    assert torch.equal(fin, S0)
    _, fin0, _ = run_gpu(d, output_final_state=True)
    assert torch.count_nonzero(fin0).item() == 0


def test_beta_zero_gives_exact_zero():
    d = to_dev(W.generate(small(B=2, T=190, H=2), 31))
    d["beta"] = torch.zeros_like(d["beta"])
    o, fin, _ = run_gpu(d, output_final_state=True)
    assert torch.count_nonzero(o).item() == 0 and torch.count_nonzero(fin).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_basis_key_table_exact(dtype):
    # g = 0, beta = 1, keys and queries are basis vectors, integer values,
    # scale 2^-3: every intermediate is an exact small integer, so the GPU
    # must match the table read-out bit for bit
    rng = np.random.default_rng(3)
    T, H = 300, 2
    widx = rng.integers(0, 128, (T, H)); qidx = rng.integers(0, 128, (T, H))
    widx[:, 1] = rng.integers(0, 6, T)                   # many rewrites of few keys
    dt = W.torch_dtype(dtype)
    eye = torch.eye(128)
    k = eye[torch.from_numpy(widx)].to(dt)[None]
    q = eye[torch.from_numpy(qidx)].to(dt)[None]
    v = torch.from_numpy(rng.integers(-8, 9, (1, T, H, 128)).astype(np.float32)).to(dt)
    d = {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV), "g": torch.zeros(1, T, H, device=DEV),
         "beta": torch.ones(1, T, H, dtype=dt, device=DEV), "scale": 0.125, "offsets": None,
         "workload": small(B=1, T=T, H=H, dtype=dtype)}
    o, _, _ = run_gpu(d)
    out = np32(o[0])
    vv = np32(v[0])
    for h in range(H):
        table = np.zeros((128, 128), np.float32)
        for t in range(T):
            table[widx[t, h]] = vv[t, h]
            assert np.array_equal(out[t, h], 0.125 * table[qidx[t, h]]), (t, h)


def test_total_forgetting():
    d = to_dev(W.generate(small(B=1, T=200, H=2), 41))
    d["g"] = torch.full_like(d["g"], -1e4)
    o, _, _ = run_gpu(d)
    q, k, v, beta = (np32(d[n][0]).astype(np.float64) for n in ("q", "k", "v", "beta"))
    ref = d["scale"] * (beta * np.einsum("thk,thk->th", q, k))[..., None] * v
    # each o_t is one product P_tt * v_new_t of two fp16-rounded operands
    # (2 * 2^-11 relative) and max|o|/rms(o) is about 8 here: about 8e-3 at most
    assert_close(np32(o[0]), ref, 1e-2, "total forgetting")


def test_orthonormal_keys_retrieve():
    # g = 0, beta = 1, an orthonormal key set (fp32 inputs): querying a key
    # written once returns its value
    rng = np.random.default_rng(8)
    Qm, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    T = 128
    k = torch.from_numpy(np.ascontiguousarray(Qm.T.astype(np.float32)))[None, :, None, :].contiguous()
    v = torch.from_numpy(rng.standard_normal((1, T, 1, 128)).astype(np.float32))
    d = {"q": k.to(DEV), "k": k.to(DEV), "v": v.to(DEV), "g": torch.zeros(1, T, 1, device=DEV),
         "beta": torch.ones(1, T, 1, device=DEV), "scale": 1.0, "offsets": None,
         "workload": small(B=1, T=T, H=1, dtype="fp32")}
    _, fin, _ = run_gpu(d, output_final_state=True)
    S = np32(fin[0, 0]).astype(np.float64)
    got = Qm.T @ S
    np.testing.assert_allclose(got, np32(v[0, :, 0]), atol=1e-4)


# ------------------------------------------------------------------ varlen
def test_varlen_packed_matches_oracle_and_separate_runs():
    lens = [1, 63, 64, 65, 200, 7, 128]
    cu = W.cu_from_lengths(lens)
    T = cu[-1]
    base = W.generate(small(B=1, T=T, H=3), 51)
    d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    d.update(scale=base["scale"], offsets=cu, workload=small(B=1, T=T, H=3, layout="TND", n_docs=len(lens)))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    assert_close(np32(o), r["o"], TOL["bf16"], "packed o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "packed final")
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        sep = {n: d[n][a:b][None].contiguous() for n in ("q", "k", "v", "g", "beta")}
        sep.update(scale=d["scale"], offsets=None, workload=small(B=1, T=b - a, H=3))
        o1, f1, _ = run_gpu(sep, output_final_state=True)
        assert torch.equal(o1[0], o[a:b]), f"document {i} differs from its separate run"
        assert torch.equal(f1[0], fin[i])


@pytest.mark.parametrize("n_docs", [1500, 2500])
def test_varlen_many_documents(n_docs):
    # many short documents: 1500 are ranked longest first over two tiles of
    # the ordering kernel; above 2048 the units keep their natural order
    rng = np.random.default_rng(n_docs)
    lens = [int(x) for x in rng.integers(1, 41, n_docs)]
    cu = W.cu_from_lengths(lens)
    T, H = cu[-1], 1
    print(f"varlen {n_docs} documents, {T} tokens", flush=True)
    base = W.generate(small(B=1, T=T, H=H), 59)
    d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    d.update(scale=base["scale"], offsets=cu, workload=small(B=1, T=T, H=H, layout="TND", n_docs=n_docs))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    assert_close(np32(o), r["o"], TOL["bf16"], "many documents o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "many documents final")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_varlen_increasing_lengths_with_entry_states(dtype):
    # documents in increasing length: the state passes launch them in the
    # reverse order, and every document's output, chunk states and final
    # state must still land in its own place
    lens = [3, 70, 129, 300]
    cu = W.cu_from_lengths(lens)
    T, H = cu[-1], 2
    print(f"varlen increasing lengths {dtype}", flush=True)
    base = W.generate(small(B=1, T=T, H=H, dtype=dtype), 53)
    d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    d.update(scale=base["scale"], offsets=cu,
             workload=small(B=1, T=T, H=H, dtype=dtype, layout="TND", n_docs=len(lens)))
    S0 = (torch.randn(len(lens), H, 128, 128, generator=torch.Generator().manual_seed(5)) * 0.3).to(DEV)
    o, fin, ex = run_gpu(d, initial_state=S0, output_final_state=True, want_h=True)
    r = run_oracle(d, S0=np32(S0).astype(np.float64), chunk_states=True)
    tol = TOL[dtype]
    assert_close(np32(o), r["o"], tol, "packed o")
    assert_close(np32(fin), r["final"], tol, "packed final")
    assert_close(np32(ex["h"]), r["chunk_states"], tol, "packed chunk entry states")


# ------------------------------------------------------------------ per-key + split
@pytest.mark.parametrize("seg", [[0, 128, 256], [0, 100, 190, 256], [0, 64, 65, 200, 256]])
def test_split_equals_unsplit_slow_decay(seg):
    # slow per-key decay keeps M far from zero, so a wrong M cannot hide
    w = small(B=2, T=256, H=2, per_key=True, use_exp2=True, gate_coef=0.001)
    d = to_dev(W.generate(w, 61 + len(seg)))
    S0 = (torch.randn(2, 2, 128, 128, device=DEV) * 0.5).contiguous()
    o_u, f_u, _ = run_gpu(d, initial_state=S0, output_final_state=True)
    o_s, f_s, S_init = gb.split_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                        seg=seg, use_exp2=True, initial_state=S0)
    torch.cuda.synchronize()
    r = run_oracle(d, S0=np32(S0).astype(np.float64))
    assert_close(np32(o_u.reshape(-1, 2, 128)), r["o"], TOL["bf16"], "unsplit o")
    assert_close(np32(o_s.reshape(-1, 2, 128)), r["o"], TOL["bf16"], "split o")
    assert_close(np32(f_s), r["final"], TOL["bf16"], "split final")
    assert_close(np32(f_u), r["final"], TOL["bf16"], "unsplit final")
    # summaries and merged entry states against the oracle
    q, k, v, g, beta = flat_inputs(d)
    offs = gb.segment_offsets(2, 256, seg)
    s = oracle.summary(k, v, g, beta, offs, gate_per_key=True, use_exp2=True)
    meta = gb.make_meta(offs, 512, DEV)
    S_ext, M, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, use_exp2=True)
    torch.cuda.synchronize()
    assert_close(np32(S_ext), s["S_ext"], TOL["bf16"], "S_ext")
    assert_close(np32(M), s["M"], TOL["bf16"], "M")
    n_seg = len(seg) - 1
    ext = s["S_ext"].reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    MM = s["M"].reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    si = oracle.merge(ext, MM, np32(S0).reshape(4, 128, 128).astype(np.float64))
    si_gpu = np32(S_init).reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    assert_close(si_gpu, si[:n_seg], TOL["bf16"], "S_init")
    # the transposed transfer map would not reproduce the unsplit end state
    wrong = oracle.merge(ext, np.swapaxes(MM, -1, -2), np32(S0).reshape(4, 128, 128).astype(np.float64))
    assert rel_err(wrong[n_seg], r["final"].reshape(4, 128, 128)) > 0.05


def test_merge_kernel_against_oracle():
    B, H, n_seg = 2, 3, 4
    g = torch.Generator().manual_seed(7)
    S_ext = torch.randn(B * n_seg, H, 128, 128, generator=g).to(DEV)
    M = (torch.randn(B * n_seg, H, 128, 128, generator=g) * 0.05).to(DEV)
    S0 = torch.randn(B, H, 128, 128, generator=g).to(DEV)
    S_init, S_final = gb.gdn_state_merge(S_ext, M, S0, B=B, n_seg=n_seg)
    torch.cuda.synchronize()
    ext = np32(S_ext).reshape(B, n_seg, H, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, B * H, 128, 128)
    MM = np32(M).reshape(B, n_seg, H, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, B * H, 128, 128)
    si = oracle.merge(ext, MM, np32(S0).reshape(B * H, 128, 128))
    got = np32(S_init).reshape(B, n_seg, H, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, B * H, 128, 128)
    assert_close(got, si[:n_seg], 1e-5, "S_init")
    assert_close(np32(S_final).reshape(B * H, 128, 128), si[n_seg], 1e-5, "S_final")


def test_per_key_small_forward():
    w = small(B=1, T=300, H=2, per_key=True, use_exp2=True, gate_coef=0.05)
    d = to_dev(W.generate(w, 71))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    assert_close(np32(o[0]), r["o"], TOL["bf16"], "per-key o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "per-key final")


@pytest.mark.parametrize("use_exp2", [False, True])
def test_per_key_fp32_with_entry_state(use_exp2):
    # fp32 inputs with a per-key gate (the fp32 preparation and state pass),
    # both decay bases, a random entry state and a ragged tail
    print(f"per-key fp32 exp2={use_exp2}", flush=True)
    w = small(B=2, T=170, H=2, dtype="fp32", per_key=True, use_exp2=use_exp2, gate_coef=0.05)
    d = to_dev(W.generate(w, 73))
    S0 = (torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(4)) * 0.3).to(DEV)
    o, fin, ex = run_gpu(d, initial_state=S0, output_final_state=True, want_h=True)
    r = run_oracle(d, S0=np32(S0).astype(np.float64), chunk_states=True)
    assert_close(flat_o(o, w), r["o"], TOL["fp32"], "per-key fp32 o")
    assert_close(np32(fin), r["final"], TOL["fp32"], "per-key fp32 final")
    assert_close(np32(ex["h"]), r["chunk_states"], TOL["fp32"], "per-key fp32 chunk states")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_per_key_packed_documents(dtype):
    # packed documents with a per-key gate: state reset per document, partial
    # chunks, against the oracle and against the separate runs (bitwise)
    lens = [40, 130, 1, 97]
    cu = W.cu_from_lengths(lens)
    T, H = cu[-1], 2
    print(f"per-key packed {dtype}", flush=True)
    base = W.generate(small(B=1, T=T, H=H, dtype=dtype, per_key=True, use_exp2=True, gate_coef=0.05), 79)
    d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    d.update(scale=base["scale"], offsets=cu,
             workload=small(B=1, T=T, H=H, dtype=dtype, per_key=True, use_exp2=True, gate_coef=0.05,
                            layout="TND", n_docs=len(lens)))
    o, fin, _ = run_gpu(d, output_final_state=True)
    r = run_oracle(d)
    assert_close(np32(o), r["o"], TOL[dtype], "per-key packed o")
    assert_close(np32(fin), r["final"], TOL[dtype], "per-key packed final")
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        sep = {n: d[n][a:b][None].contiguous() for n in ("q", "k", "v", "g", "beta")}
        sep.update(scale=d["scale"], offsets=None,
                   workload=small(B=1, T=b - a, H=H, dtype=dtype, per_key=True, use_exp2=True))
        o1, f1, _ = run_gpu(sep, output_final_state=True)
        assert torch.equal(o1[0], o[a:b]), f"document {i} differs from its separate run"
        assert torch.equal(f1[0], fin[i])


# ------------------------------------------------------------------ full-size workloads (sampled)
def _sampled_check(d, o, heads, fin=None):
    """Oracle on the selected heads only (heads are independent)."""
    w = d["workload"]

    def pick(x):
        x = x.reshape(-1, *x.shape[2:]) if w.layout == "BSND" else x
        return np32(x[:, heads].contiguous())

    q, k, v, g, beta = (pick(d[n]) for n in ("q", "k", "v", "g", "beta"))
    r = oracle.fwd(q, k, v, g, beta, unit_offsets(d), d["scale"], gate_per_key=w.gate_per_key,
                   use_exp2=w.use_exp2, want_final=fin is not None)
    e = assert_close(pick(o), r["o"], TOL[w.dtype], f"{w.name} o (heads {heads})")
    if fin is not None:
        assert_close(np32(fin[:, heads]), r["final"], TOL[w.dtype], f"{w.name} final")
    return e


def test_workload_dense_bf16_full():
    w = W.WORKLOADS[1]
    d = W.generate(w, 1001, device=DEV)
    o, _, _ = run_gpu(d)
    e = _sampled_check(d, o, heads=[0, 7, 15])
    print(f"{w.name}: sampled o err/rms {e:.2e}")


def test_workload_varlen_full():
    w = W.WORKLOADS[2]
    d = W.generate(w, 1002, device=DEV)
    o, fin, _ = run_gpu(d, output_final_state=True)
    e = _sampled_check(d, o, heads=[3, 30], fin=fin)
    print(f"{w.name}: sampled o err/rms {e:.2e}")


def test_workload_kda_split_full():
    w = W.WORKLOADS[3]
    d = W.generate(w, 1003, device=DEV)
    o_s, f_s, _ = gb.split_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                   seg=d["seg_offsets"], use_exp2=True)
    o_u, f_u, _ = run_gpu(d, output_final_state=True)
    torch.cuda.synchronize()
    # split == unsplit on the GPU, and both against the oracle on sampled heads
    assert_close(np32(o_s.reshape(-1, 8, 128)), np32(o_u.reshape(-1, 8, 128)), TOL["bf16"], "split vs unsplit")
    d2 = dict(d)
    d2["offsets"] = [0, w.T, 2 * w.T]
    e = _sampled_check(d2, o_s, heads=[1, 6], fin=f_s)
    print(f"{w.name}: sampled split o err/rms {e:.2e}")


def test_workload_long_full():
    w = W.WORKLOADS[4]
    d = W.generate(w, 1004, device=DEV)
    o, fin, _ = run_gpu(d, output_final_state=True)
    e = _sampled_check(d, o, heads=[5], fin=fin)
    print(f"{w.name}: sampled o err/rms {e:.2e}")


# ------------------------------------------------------------------ strong per-key gates
def _no_nan(*ts):
    for t in ts:
        assert torch.isfinite(t).all(), "non-finite values in the output"


@pytest.mark.parametrize("coef", [0.6, 1.0, 4.0])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_per_key_strong_gates(coef, dtype):
    # g = -coef softplus(N(0,1)) per key in log2 units: up to tens of log2
    # units of decay inside one 16-token block, which the factored fp16
    # operands of the L and P tiles must survive (and the direct diagonal
    # tiles take over from); ragged tail, entry state, chunk states
    print(f"per-key strong gate coef={coef} {dtype}", flush=True)
    w = small(B=2, T=200, H=2, dtype=dtype, per_key=True, use_exp2=True, gate_coef=coef)
    d = to_dev(W.generate(w, 131 + int(10 * coef)))
    S0 = (torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(13)) * 0.3).to(DEV)
    o, fin, ex = run_gpu(d, initial_state=S0, output_final_state=True, want_h=True)
    _no_nan(o, fin, ex["h"])
    r = run_oracle(d, S0=np32(S0).astype(np.float64), chunk_states=True)
    tol = TOL[dtype]
    assert_close(flat_o(o, w), r["o"], tol, "strong-gate o")
    assert_close(np32(fin), r["final"], tol, "strong-gate final")
    assert_close(np32(ex["h"]), r["chunk_states"], tol, "strong-gate chunk states")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_per_key_total_forgetting(dtype):
    # g = -1e4 on every key: each token sees only its own write, so
    # o_t = scale beta_t (q_t . k_t) v_t, and the final state is
    # beta_T k_T v_T^T of the last token
    print(f"per-key total forgetting {dtype}", flush=True)
    T, H = 200, 2
    d = to_dev(W.generate(small(B=1, T=T, H=H, dtype=dtype, per_key=True, use_exp2=True), 43))
    d["g"] = torch.full_like(d["g"], -1e4)
    o, fin, _ = run_gpu(d, output_final_state=True)
    _no_nan(o, fin)
    q, k, v, beta = (np32(d[n][0]).astype(np.float64) for n in ("q", "k", "v", "beta"))
    ref = d["scale"] * (beta * np.einsum("thk,thk->th", q, k))[..., None] * v
    fref = beta[-1][:, None, None] * np.einsum("hk,hv->hkv", k[-1], v[-1])
    # bf16: one product P_tt v_new_t of two fp16-rounded operands per token
    # (2 * 2^-11 relative; max|o|/rms(o) is about 8): 1e-2
    tol = 1e-2 if dtype == "bf16" else TOL["fp32"]
    assert_close(np32(o[0]), ref, tol, "per-key total forgetting o")
    assert_close(np32(fin[0]), fref, tol, "per-key total forgetting final")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_split_strong_per_key_gates(dtype):
    # summary -> merge -> correction with strong per-key gates (coef 1, log2):
    # the transfer maps are tiny but must be finite, and split == oracle
    print(f"split with strong per-key gates {dtype}", flush=True)
    w = small(B=2, T=256, H=2, dtype=dtype, per_key=True, use_exp2=True, gate_coef=1.0)
    d = to_dev(W.generate(w, 149))
    seg = [0, 64, 150, 256]
    S0 = (torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(3)) * 0.5).to(DEV)
    o_s, f_s, S_init = gb.split_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], seg=seg,
                                        use_exp2=True, initial_state=S0)
    torch.cuda.synchronize()
    _no_nan(o_s, f_s, S_init)
    r = run_oracle(d, S0=np32(S0).astype(np.float64))
    assert_close(flat_o(o_s, w), r["o"], TOL[dtype], "split o")
    assert_close(np32(f_s), r["final"], TOL[dtype], "split final")


# ------------------------------------------------------------------ every summary path
def _split_case(per_key, dtype, seed):
    # slow decay keeps the transfer map far from zero, so a wrong M cannot hide
    if per_key:
        w = small(B=2, T=256, H=2, dtype=dtype, per_key=True, use_exp2=True, gate_coef=0.001)
    else:
        w = small(B=2, T=256, H=2, dtype=dtype, gate_coef=0.002)
    return w, to_dev(W.generate(w, seed))


@pytest.mark.parametrize("seg", [[0, 128, 256], [0, 100, 190, 256], [0, 64, 65, 200, 256]])
@pytest.mark.parametrize("per_key,dtype", [(False, "bf16"), (False, "fp32"), (True, "fp32")])
def test_split_equals_unsplit_every_path(seg, per_key, dtype):
    # the summary kernels not covered by the bf16 per-key case above: the
    # scalar-gate summary (bf16 and fp32) and the fp32 per-key summary;
    # non-symmetric entry state, aligned and unaligned cuts
    print(f"split path per_key={per_key} {dtype} seg={seg}", flush=True)
    w, d = _split_case(per_key, dtype, 167 + len(seg))
    tol = TOL[dtype]
    S0 = (torch.randn(2, 2, 128, 128, generator=torch.Generator().manual_seed(19)) * 0.5).to(DEV)
    ue2 = w.use_exp2
    o_s, f_s, S_init = gb.split_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], seg=seg,
                                        use_exp2=ue2, initial_state=S0)
    torch.cuda.synchronize()
    r = run_oracle(d, S0=np32(S0).astype(np.float64))
    assert_close(flat_o(o_s, w), r["o"], tol, "split o")
    assert_close(np32(f_s), r["final"], tol, "split final")
    q, k, v, g, beta = flat_inputs(d)
    offs = gb.segment_offsets(2, 256, seg)
    s = oracle.summary(k, v, g, beta, offs, gate_per_key=per_key, use_exp2=ue2)
    meta = gb.make_meta(offs, 512, DEV)
    S_ext, M, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, use_exp2=ue2)
    torch.cuda.synchronize()
    assert_close(np32(S_ext), s["S_ext"], tol, "S_ext")
    assert_close(np32(M), s["M"], tol, "M")
    n_seg = len(seg) - 1
    ext = s["S_ext"].reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    MM = s["M"].reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    si = oracle.merge(ext, MM, np32(S0).reshape(4, 128, 128).astype(np.float64))
    si_gpu = np32(S_init).reshape(2, n_seg, 2, 128, 128).transpose(1, 0, 2, 3, 4).reshape(n_seg, 4, 128, 128)
    assert_close(si_gpu, si[:n_seg], tol, "S_init")
    # a transposed transfer map does not reproduce the unsplit end state
    wrong = oracle.merge(ext, np.swapaxes(MM, -1, -2), np32(S0).reshape(4, 128, 128).astype(np.float64))
    assert rel_err(wrong[n_seg], r["final"].reshape(4, 128, 128)) > 0.05


@pytest.mark.parametrize("per_key,dtype", [(False, "bf16"), (True, "bf16"), (False, "fp32"), (True, "fp32")])
def test_summary_modes(per_key, dtype):
    # mode 1 (S_ext only) and mode 2 (M only) each equal their half of mode 0
    # bit for bit (the same column tiles of the same recurrence), and match
    # the oracle
    print(f"summary modes per_key={per_key} {dtype}", flush=True)
    w, d = _split_case(per_key, dtype, 181)
    offs = gb.segment_offsets(2, 256, [0, 100, 256])
    meta = gb.make_meta(offs, 512, DEV)
    kw = dict(meta=meta, use_exp2=w.use_exp2)
    e0, m0, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], mode=0, **kw)
    e1, m1, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], mode=1, **kw)
    e2, m2, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], mode=2, **kw)
    torch.cuda.synchronize()
    assert m1 is None and e2 is None
    assert torch.equal(e1, e0), "mode 1 S_ext differs from mode 0"
    assert torch.equal(m2, m0), "mode 2 M differs from mode 0"
    q, k, v, g, beta = flat_inputs(d)
    s = oracle.summary(k, v, g, beta, offs, gate_per_key=per_key, use_exp2=w.use_exp2)
    assert_close(np32(e1), s["S_ext"], TOL[dtype], "mode 1 S_ext")
    assert_close(np32(m2), s["M"], TOL[dtype], "mode 2 M")


@pytest.mark.parametrize("per_key", [False, True])
def test_values_near_the_fp16_operand_range(per_key):
    # bf16 inputs become fp16 operands, and the state, the residual and v_new
    # are rounded to fp16 every chunk: with v scaled by 2^11 (|v| up to about
    # 1e4, the state and v_new alike) every operand stays inside fp16's range
    # and the relative error is that of unit-scale inputs
    print(f"values near the fp16 range per_key={per_key}", flush=True)
    w = small(B=1, T=300, H=2, per_key=per_key, use_exp2=per_key, gate_coef=0.05 if per_key else 0.1)
    d = to_dev(W.generate(w, 191))
    d["v"] = (d["v"].float() * 2048.0).to(torch.bfloat16)
    S0 = (torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(2)) * 2048.0).to(DEV)
    o, fin, _ = run_gpu(d, initial_state=S0, output_final_state=True)
    _no_nan(o, fin)
    assert float(d["v"].float().abs().max()) > 8000.0
    r = run_oracle(d, S0=np32(S0).astype(np.float64))
    assert_close(flat_o(o, w), r["o"], TOL["bf16"], "scaled o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "scaled final")


@pytest.mark.parametrize("per_key,dtype,with_final", [(False, "bf16", True), (True, "bf16", False), (False, "fp32", False)])
def test_pieced_forward_equals_one_pass(per_key, dtype, with_final):
    # a long row with two heads (8 state workgroups) runs in pieces whose
    # preparations overlap the state pass; bit for bit the one-pass forward
    # (prepare, then reuse, which never runs in pieces), and the oracle on a
    # sampled head
    print(f"pieced forward per_key={per_key} {dtype} final={with_final}", flush=True)
    T = 16384 + 37
    w = small(B=1, T=T, H=2, dtype=dtype, per_key=per_key, use_exp2=per_key, gate_coef=0.02 if per_key else 0.1)
    d = to_dev(W.generate(w, 611))
    S0 = (torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(612)) * 0.3).to(DEV)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"])
    o1, f1, ex1 = gb.gdn_chunk_fwd(*args, initial_state=S0, output_final_state=with_final, use_exp2=w.use_exp2,
                                   slots=("v_new",))
    nb = gb.workspace_bytes(gb._desc(d["k"], 2, d["k"].dtype, torch.float32, per_key, w.use_exp2, d["scale"], None))
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    gb.gdn_chunk_fwd(d["q"], d["k"], None, d["g"], d["beta"], d["scale"], use_exp2=w.use_exp2,
                     flags=gb.FLAG_PREPARE_ONLY, workspace=ws)
    o2, f2, ex2 = gb.gdn_chunk_fwd(*args, initial_state=S0, output_final_state=with_final, use_exp2=w.use_exp2,
                                   flags=gb.FLAG_REUSE_PREPARED, workspace=ws, slots=("v_new",))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "pieced o differs from the one-pass o"
    assert torch.equal(ex1["v_new"], ex2["v_new"])
    if with_final:
        assert torch.equal(f1, f2)
    q, k, v, g, beta = flat_inputs(d)
    pick = lambda x: np.ascontiguousarray(x[:, [1]])
    r = oracle.fwd(pick(q), pick(k), pick(v), pick(g), pick(beta), [0, T], d["scale"], gate_per_key=per_key,
                   use_exp2=w.use_exp2, S0=np32(S0)[:, [1]].astype(np.float64))
    assert_close(flat_o(o1, w)[:, [1]], r["o"], TOL[dtype], "pieced o (head 1)")
    if with_final:
        assert_close(np32(f1[:, [1]]), r["final"], TOL[dtype], "pieced final (head 1)")


def test_long_row_forward_under_graph_capture():
    # a row long enough for the pieced forward, captured into a graph on a
    # side stream: under capture the forward runs its single pass on the
    # capturing stream (no helper stream joins the graph); every replay,
    # with eager work and synchronisations between them, gives the bits of
    # the eager (pieced) call
    print("long-row forward under graph capture", flush=True)
    T = 16384 + 37
    w = small(B=1, T=T, H=2, dtype="bf16")
    d = to_dev(W.generate(w, 613))
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"])
    nb = gb.workspace_bytes(gb._desc(d["k"], 2, d["k"].dtype, torch.float32, False, False, d["scale"], None))
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o = torch.empty(d["v"].shape, dtype=torch.float32, device=DEV)
    fin = torch.empty((1, 2, 128, 128), dtype=torch.float32, device=DEV)
    o_e, f_e, _ = gb.gdn_chunk_fwd(*args, output_final_state=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gb.gdn_chunk_fwd(*args, output_final_state=True, workspace=ws, out=o, final_out=fin)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(fin, f_e), f"replay {rep}"
