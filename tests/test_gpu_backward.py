"""Parity of the HIP backward (gdn_chunk_bwd, through the C ABI) with the fp64
backward oracle. Tolerances as for the forward, per gradient: max |x - ref|
<= tol * rms(ref), tol = 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs); dL/do is
drawn in fp32 and rounded to the input dtype, and the oracle sees the same
rounded values."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_05_amd import binding as gb
from chunked_gated_delta_05_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, flat_inputs, np32, unit_offsets

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("dq", "dk", "dv", "dg", "dbeta")


def small(B=1, T=200, H=3, dtype="bf16", use_exp2=False, gate_coef=0.1, layout="BSND", n_docs=0, per_key=False):
    return W.Workload("small", B=B, T=T, H=H, dtype=dtype, layout=layout, use_exp2=use_exp2,
                      gate_coef=gate_coef, n_docs=n_docs, gate_per_key=per_key)


def packed(lens, H, dtype, seed, per_key=False):
    cu = W.cu_from_lengths(lens)
    kw = dict(use_exp2=per_key, gate_coef=0.05 if per_key else 0.1, per_key=per_key)
    base = W.generate(small(B=1, T=cu[-1], H=H, dtype=dtype, **kw), seed)
    d = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    d.update(scale=base["scale"], offsets=cu,
             workload=small(B=1, T=cu[-1], H=H, dtype=dtype, layout="TND", n_docs=len(lens), **kw))
    return d


def run_both(d, seed, S0=False, dht=False, heads=None):
    """GPU forward (entry states) + backward, and the oracle's backward on the
    same rounded inputs (restricted to `heads` when given)."""
    w = d["workload"]
    dev = {n: d[n] if d[n].is_cuda else d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}
    meta = gb.make_meta(d["offsets"], w.T, DEV) if w.layout == "TND" else None
    offs = unit_offsets(d)
    units = len(offs) - 1
    gen = torch.Generator().manual_seed(seed)
    s0 = (torch.randn(units, w.H, 128, 128, generator=gen) * 0.3).to(DEV) if S0 else None
    dh = (torch.randn(units, w.H, 128, 128, generator=gen) * 0.3).to(DEV) if dht else None
    do = torch.randn(dev["v"].shape, generator=gen).to(dev["v"].dtype).to(DEV)
    _, _, ex = gb.gdn_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], d["scale"], meta=meta,
                                initial_state=s0, use_exp2=w.use_exp2, want_h=True)
    got = gb.gdn_chunk_bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], ex["h"], do, d["scale"], meta=meta,
                           dht=dh, use_exp2=w.use_exp2)
    torch.cuda.synchronize()
    q, k, v, g, beta = flat_inputs(d)
    flat = (lambda x: x.reshape(-1, *x.shape[2:])) if w.layout == "BSND" else (lambda x: x)
    dof = np32(flat(do))
    sel = slice(None) if heads is None else heads
    pick = lambda x: np.ascontiguousarray(x[:, sel])
    ref = oracle.bwd(pick(q), pick(k), pick(v), pick(g), pick(beta), offs, d["scale"], pick(dof),
                     gate_per_key=w.gate_per_key, use_exp2=w.use_exp2,
                     S0=None if s0 is None else np32(s0)[:, sel].astype(np.float64),
                     dht=None if dh is None else np32(dh)[:, sel].astype(np.float64))
    out = {n: pick(np32(flat(got[n]))) for n in NAMES}
    out["dh0"] = np32(got["dh0"])[:, sel]
    return out, ref


def check_all(out, ref, tol, what):
    errs = {}
    for n in NAMES + ("dh0",):
        ref_n = ref["dS0"] if n == "dh0" else ref[n]
        errs[n] = assert_close(out[n], ref_n, tol, f"{what} {n}")
    return errs


@pytest.mark.parametrize("B,T,H", [(1, 64, 1), (2, 200, 3), (1, 1, 2), (1, 130, 2), (3, 63, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_small(B, T, H, dtype):
    print(f"backward B={B} T={T} H={H} {dtype}", flush=True)
    d = W.generate(small(B=B, T=T, H=H, dtype=dtype), 211 + T)
    out, ref = run_both(d, 5 + T, S0=True, dht=True)
    check_all(out, ref, TOL[dtype], "small")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_base2_gate(dtype):
    print(f"backward base-2 gate {dtype}", flush=True)
    d = W.generate(small(B=2, T=150, H=2, dtype=dtype, use_exp2=True, gate_coef=0.05), 223)
    out, ref = run_both(d, 7, S0=True, dht=True)
    check_all(out, ref, TOL[dtype], "base 2")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_packed_documents(dtype):
    # packed documents with ragged chunks, an entry state and dL/dh_final per document
    print(f"backward packed {dtype}", flush=True)
    d = packed([1, 63, 64, 65, 200, 7, 128], 3, dtype, 227)
    out, ref = run_both(d, 9, S0=True, dht=True)
    check_all(out, ref, TOL[dtype], "packed")


def test_backward_beta_zero_is_exactly_zero():
    # beta = 0 and no entry state keep h = 0: dq, dk, dv and dg are exactly
    # zero on the GPU as in the oracle; dbeta matches the oracle
    print("backward beta = 0", flush=True)
    d = W.generate(small(B=1, T=150, H=2), 229)
    d["beta"] = torch.zeros_like(d["beta"])
    out, ref = run_both(d, 11)
    for n in ("dq", "dk", "dv", "dg"):
        assert np.count_nonzero(out[n]) == 0, n
    assert_close(out["dbeta"], ref["dbeta"], TOL["bf16"], "dbeta")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_total_forgetting(dtype):
    print(f"backward total forgetting {dtype}", flush=True)
    d = W.generate(small(B=1, T=140, H=2, dtype=dtype), 233)
    d["g"] = torch.full_like(d["g"], -1e4)
    out, ref = run_both(d, 13, dht=True)
    for n in NAMES:
        assert np.isfinite(out[n]).all(), n
    check_all({n: out[n] for n in ("dq", "dk", "dv", "dbeta", "dh0")} | {"dg": ref["dg"]}, ref, TOL[dtype],
              "total forgetting")
    assert np.abs(out["dg"]).max() <= 1e-6 * max(1.0, np.abs(out["dq"]).max())


@pytest.mark.parametrize("coef", [1.0, 4.0])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_strong_scalar_gates(coef, dtype):
    # strong scalar decays (g = -c softplus, base e): products of decays reach
    # e^-180 inside a chunk, below fp16's range, so the chunk maps of the
    # bf16 path lose them to underflow; every gradient finite and at the
    # oracle within the plain bars (measured at c = 4: bf16 dv 1.6e-2, dk
    # 1.4e-2 of rms; fp32 dg 4.8e-5)
    print(f"backward strong scalar gate c={coef} {dtype}", flush=True)
    d = W.generate(small(B=1, T=200, H=2, dtype=dtype, gate_coef=coef), 271)
    out, ref = run_both(d, 25, S0=True, dht=True)
    for n in NAMES + ("dh0",):
        assert np.isfinite(out[n]).all(), n
    check_all(out, ref, TOL[dtype], f"scalar c={coef}")


def test_backward_tiny_fp32_workload():
    w = W.WORKLOADS[0]
    d = W.generate(w, 1000)
    out, ref = run_both(d, 15, dht=True)
    errs = check_all(out, ref, TOL["fp32"], w.name)
    print(f"{w.name} backward: " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))


def test_backward_dense_bf16_workload_sampled_heads():
    w = W.WORKLOADS[1]
    d = W.generate(w, 1001, device=DEV)
    out, ref = run_both(d, 17, heads=[0, 9])
    errs = check_all(out, ref, TOL["bf16"], w.name)
    print(f"{w.name} backward (heads 0, 9): " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))


def test_autograd_op_matches_the_abi():
    # GatedDeltaRule: forward output and final state as gdn_chunk_fwd, and its
    # backward (dL/do and dL/d final) returns gdn_chunk_bwd's gradients
    d = W.generate(small(B=2, T=130, H=2, dtype="fp32"), 239)
    x = {n: d[n].to(DEV).requires_grad_(n != "g" or True) for n in ("q", "k", "v", "g", "beta")}
    s0 = (torch.randn(2, 2, 128, 128) * 0.3).to(DEV).requires_grad_(True)
    o, fin = gb.GatedDeltaRule.apply(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, d["scale"])
    do = torch.randn_like(o)
    (o * do).sum().backward()
    _, _, ex = gb.gdn_chunk_fwd(*(x[n].detach() for n in ("q", "k", "v", "g", "beta")), d["scale"],
                                initial_state=s0.detach(), want_h=True)
    r = gb.gdn_chunk_bwd(*(x[n].detach() for n in ("q", "k", "v", "g", "beta")), ex["h"], do, d["scale"])
    torch.cuda.synchronize()
    for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta")):
        assert torch.equal(x[t].grad, r[n]), n
    assert torch.equal(s0.grad, r["dh0"])


def test_backward_is_deterministic():
    # no float atomics in any reduction: two calls give the same bits
    d = W.generate(small(B=2, T=300, H=3), 241)
    x = {n: d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}
    _, _, ex = gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], d["scale"], want_h=True)
    do = torch.randn(x["v"].shape, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    r1 = gb.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], ex["h"], do, d["scale"])
    r2 = gb.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], ex["h"], do, d["scale"])
    torch.cuda.synchronize()
    for n in r1:
        assert torch.equal(r1[n], r2[n]), n


@pytest.mark.parametrize("per_key", [False, True])
def test_backward_reusing_the_preparation(per_key):
    # a backward that reuses the preparation a gradient summary left in the
    # workspace gives the bits of one that prepares itself
    w = small(B=2, T=200, H=2, use_exp2=per_key, gate_coef=0.05, per_key=per_key)
    d = W.generate(w, 281)
    x = [d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")]
    meta = gb.make_meta([0, 200, 400], 400, DEV)
    xf = [t.reshape(-1, *t.shape[2:]) for t in x]
    _, _, ex = gb.gdn_chunk_fwd(*xf, d["scale"], meta=meta, want_h=True, use_exp2=per_key)
    do = torch.randn(xf[2].shape, generator=torch.Generator().manual_seed(7)).to(xf[2].dtype).to(DEV)
    r1 = gb.gdn_chunk_bwd(*xf, ex["h"], do, d["scale"], meta=meta, use_exp2=per_key)
    nb = gb.workspace_bytes_bwd(xf[1], xf[3], meta, use_exp2=per_key)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    gb.gdn_state_grad_summary(*xf, ex["h"], do, d["scale"], meta=meta, use_exp2=per_key, workspace=ws)
    r2 = gb.gdn_chunk_bwd(*xf, ex["h"], do, d["scale"], meta=meta, use_exp2=per_key, workspace=ws,
                          reuse_prepared=True)
    torch.cuda.synchronize()
    for n in r1:
        assert torch.equal(r1[n], r2[n]), n


# ------------------------------------------------------------------ per-key gate
@pytest.mark.parametrize("B,T,H,dtype,use_exp2", [(2, 150, 2, "bf16", True), (1, 130, 2, "fp32", True),
                                                  (1, 64, 1, "fp32", False), (1, 1, 2, "bf16", True),
                                                  (3, 63, 1, "bf16", False), (1, 200, 3, "fp32", False)])
def test_backward_per_key(B, T, H, dtype, use_exp2):
    print(f"per-key backward B={B} T={T} H={H} {dtype} exp2={use_exp2}", flush=True)
    w = small(B=B, T=T, H=H, dtype=dtype, use_exp2=use_exp2, gate_coef=0.05 if use_exp2 else 0.03, per_key=True)
    d = W.generate(w, 251 + T)
    out, ref = run_both(d, 19 + T, S0=True, dht=True)
    check_all(out, ref, TOL[dtype], "per key")


@pytest.mark.parametrize("H", [12, 24])
def test_backward_per_key_wide_column_tiles(H):
    # 4 x H (unit, head) pairs: with 256 compute units the per-key reverse
    # pass runs 32-column tiles at H = 12 and 64-column tiles at H = 24 (the
    # small cases above take 16-column tiles); the oracle checks two heads
    print(f"per-key backward, wide tiles: B=4 T=70 H={H}", flush=True)
    w = small(B=4, T=70, H=H, dtype="bf16", use_exp2=True, gate_coef=0.05, per_key=True)
    d = W.generate(w, 977 + H)
    out, ref = run_both(d, 31 + H, S0=True, dht=True, heads=[0, H - 1])
    check_all(out, ref, TOL["bf16"], f"per key H={H}")


@pytest.mark.parametrize("coef", [0.6, 1.0, 4.0])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_per_key_strong_gates(coef, dtype):
    # per-key decays far past the half-chunk range a middle-row factoring
    # could hold (log2 units): every gradient finite and at the oracle.
    # dg with fp32 inputs is held to 1e-4 * max(1, c): with g = -c softplus
    # (log2) the cumulative gate reaches about 50 c inside a chunk, and its
    # fp32 rounding (half an ulp of that) is what dg is most sensitive to;
    # a one-ulp change of the raw gates alone moves the exact dg by 9e-6 of
    # its rms at c = 4 against 2.6e-6 at c = 1 (fp64 oracle)
    print(f"per-key backward strong gate c={coef} {dtype}", flush=True)
    w = small(B=1, T=200, H=2, dtype=dtype, use_exp2=True, gate_coef=coef, per_key=True)
    d = W.generate(w, 257)
    out, ref = run_both(d, 21, S0=True, dht=True)
    for n in NAMES + ("dh0",):
        assert np.isfinite(out[n]).all(), n
    check_all({n: out[n] for n in NAMES + ("dh0",) if n != "dg"} | {"dg": ref["dg"]}, ref, TOL[dtype],
              f"per key c={coef}")
    tol_dg = TOL[dtype] * (max(1.0, coef) if dtype == "fp32" else 1.0)
    assert_close(out["dg"], ref["dg"], tol_dg, f"per key c={coef} dg")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_per_key_total_forgetting(dtype):
    # g = -1e4 on every key: nothing crosses a token, dg vanishes
    print(f"per-key backward total forgetting {dtype}", flush=True)
    d = W.generate(small(B=1, T=140, H=2, dtype=dtype, use_exp2=True, per_key=True), 263)
    d["g"] = torch.full_like(d["g"], -1e4)
    out, ref = run_both(d, 23, dht=True)
    for n in NAMES:
        assert np.isfinite(out[n]).all(), n
    check_all({n: out[n] for n in ("dq", "dk", "dv", "dbeta", "dh0")} | {"dg": ref["dg"]}, ref, TOL[dtype],
              "per-key total forgetting")
    assert np.abs(out["dg"]).max() <= 1e-6 * max(1.0, np.abs(out["dq"]).max())


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_per_key_packed_documents(dtype):
    print(f"per-key backward packed {dtype}", flush=True)
    d = packed([1, 63, 64, 65, 200, 7, 128], 2, dtype, 269, per_key=True)
    out, ref = run_both(d, 25, S0=True, dht=True)
    check_all(out, ref, TOL[dtype], "per-key packed")


def test_backward_per_key_segment_shape_sampled_heads():
    # one segment of the per-key split workload (B=2, 8192 tokens, 8 heads,
    # log2 gate c = 0.05, bf16), heads 1 and 6 against the oracle
    w = small(B=2, T=8192, H=8, dtype="bf16", use_exp2=True, gate_coef=0.05, per_key=True)
    d = W.generate(w, 271, device=DEV)
    out, ref = run_both(d, 27, heads=[1, 6])
    errs = check_all(out, ref, TOL["bf16"], "per-key segment")
    print("per-key segment backward (heads 1, 6): " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))


def test_backward_per_key_is_deterministic():
    w = small(B=2, T=300, H=2, use_exp2=True, gate_coef=0.05, per_key=True)
    d = W.generate(w, 277)
    x = {n: d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}
    _, _, ex = gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], d["scale"], want_h=True, use_exp2=True)
    do = torch.randn(x["v"].shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    r1 = gb.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], ex["h"], do, d["scale"], use_exp2=True)
    r2 = gb.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], ex["h"], do, d["scale"], use_exp2=True)
    torch.cuda.synchronize()
    for n in r1:
        assert torch.equal(r1[n], r2[n]), n


# ------------------------------------------------------------------ split backward
@pytest.mark.parametrize("dtype,with_dht,per_key", [("bf16", False, False), ("fp32", True, False),
                                                    ("bf16", True, False), ("bf16", True, True),
                                                    ("fp32", False, True)])
def test_split_backward_equals_unsplit(dtype, with_dht, per_key):
    # rows cut at 100 and 190 (inside chunks): gradient summaries of the
    # segments, the adjoint merge with the forward's transfer maps, then
    # every segment's backward from its exit gradient give the unsplit
    # backward, and the oracle's
    print(f"split backward {dtype} dht={with_dht} per_key={per_key}", flush=True)
    B, T, H = 2, 256, 2
    w = small(B=B, T=T, H=H, dtype=dtype, gate_coef=0.01 if per_key else 0.02, per_key=per_key, use_exp2=per_key)
    d = W.generate(w, 777)
    dev = {n: d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}
    gen = torch.Generator().manual_seed(778)
    S0 = (torch.randn(B, H, 128, 128, generator=gen) * 0.3).to(DEV)
    dht = (torch.randn(B, H, 128, 128, generator=gen) * 0.3).to(DEV) if with_dht else None
    do = torch.randn(dev["v"].shape, generator=gen).to(dev["v"].dtype).to(DEV)
    seg = [0, 100, 190, T]
    n_seg = len(seg) - 1
    meta = gb.make_meta(gb.segment_offsets(B, T, seg), B * T, DEV)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"])
    e2 = w.use_exp2
    S_ext, M, _ = gb.gdn_state_summary(dev["k"], dev["v"], dev["g"], dev["beta"], meta=meta, use_exp2=e2,
                                       q=dev["q"])
    S_init, _ = gb.gdn_state_merge(S_ext, M, S0, B=B, n_seg=n_seg, want_final=False)
    _, _, ex = gb.gdn_chunk_fwd(*args, d["scale"], meta=meta, initial_state=S_init, want_h=True, use_exp2=e2)
    got = gb.split_backward(*args, ex["h"], do, d["scale"], seg=seg, M=M, dht=dht, use_exp2=e2)
    _, _, exu = gb.gdn_chunk_fwd(*args, d["scale"], initial_state=S0, want_h=True, use_exp2=e2)
    ref_gpu = gb.gdn_chunk_bwd(*args, exu["h"], do, d["scale"], dht=dht, use_exp2=e2)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for n in NAMES + ("dh0",):
        assert_close(np32(got[n]), np32(ref_gpu[n]), tol, f"split vs unsplit {n}")
    q, k, v, g, beta = flat_inputs(d)
    flat = lambda x: x.reshape(-1, *x.shape[2:])
    ref = oracle.bwd(q, k, v, g, beta, [0, T, 2 * T], d["scale"], np32(flat(do)), gate_per_key=per_key,
                     use_exp2=e2, S0=np32(S0).astype(np.float64),
                     dht=None if dht is None else np32(dht).astype(np.float64))
    for n in NAMES:
        assert_close(np32(flat(got[n])), ref[n], tol, f"split vs oracle {n}")
    assert_close(np32(got["dh0"]), ref["dS0"], tol, "split vs oracle dh0")


@pytest.mark.parametrize("per_key", [False, True])
def test_gradient_summary_against_oracle(per_key):
    # every segment's dL/d(entry state) through its own outputs only
    print(f"gradient summary per_key={per_key}", flush=True)
    B, T, H = 1, 300, 2
    w = small(B=B, T=T, H=H, dtype="fp32", gate_coef=0.05, per_key=per_key, use_exp2=per_key)
    d = W.generate(w, 790)
    dev = {n: d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}
    gen = torch.Generator().manual_seed(791)
    do = torch.randn(dev["v"].shape, generator=gen).to(DEV)
    S_in = (torch.randn(3, H, 128, 128, generator=gen) * 0.3).to(DEV)
    offs = [0, 64, 65, 300]
    meta = gb.make_meta(offs, T, DEV)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"])
    _, _, ex = gb.gdn_chunk_fwd(*args, d["scale"], meta=meta, initial_state=S_in, want_h=True, use_exp2=per_key)
    dS = gb.gdn_state_grad_summary(*args, ex["h"], do, d["scale"], meta=meta, use_exp2=per_key)
    torch.cuda.synchronize()
    q, k, v, g, beta = flat_inputs(d)
    ref = oracle.bwd(q, k, v, g, beta, offs, d["scale"], np32(do.reshape(-1, H, 128)), gate_per_key=per_key,
                     use_exp2=per_key, S0=np32(S_in).astype(np.float64))
    assert_close(np32(dS), ref["dS0"], TOL["fp32"], "local dS")


@pytest.mark.parametrize("with_final,with_dS0", [(False, False), (True, True), (False, True)])
def test_merge_adjoint_kernel_against_oracle(with_final, with_dS0):
    # maps that must not be read (the last segment's without a final-state
    # gradient, the first's without dS0) hold NaN
    print(f"adjoint merge final={with_final} dS0={with_dS0}", flush=True)
    B, H, n_seg = 2, 3, 4
    gen = torch.Generator().manual_seed(17)
    E = torch.randn(B * n_seg, H, 128, 128, generator=gen)
    M = torch.randn(B * n_seg, H, 128, 128, generator=gen) * 0.05
    F = torch.randn(B, H, 128, 128, generator=gen) if with_final else None
    Mg = M.clone()
    for b in range(B):
        if not with_final:
            Mg[b * n_seg + n_seg - 1] = float("nan")
        if not with_dS0:
            Mg[b * n_seg] = float("nan")
    exits, dS0 = gb.gdn_state_merge_adjoint(E.to(DEV), Mg.to(DEV), None if F is None else F.to(DEV), B=B, n_seg=n_seg,
                                            want_dS0=with_dS0)
    torch.cuda.synchronize()
    for b in range(B):
        rows = slice(b * n_seg, (b + 1) * n_seg)
        want_exits, want_G0 = oracle.merge_adjoint(E[rows].numpy(), M[rows].numpy(), None if F is None else F[b].numpy())
        got = np32(exits[rows])
        assert np.isfinite(got).all()
        assert_close(got, want_exits, 1e-5, "dS_exit")
        if with_dS0:
            assert_close(np32(dS0[b]), want_G0, 1e-5, "dS0")


# ------------------------------------------------------------------ full workloads, sampled heads
def _bwd_sampled(d, got, do, heads, offs, dht=None):
    """The oracle's backward on the given heads only (sliced on the GPU
    before the copy), against the GPU gradients of those heads."""
    w = d["workload"]
    flat = (lambda x: x.reshape(-1, *x.shape[2:])) if w.layout == "BSND" else (lambda x: x)
    sel = lambda x: np32(flat(x)[:, heads].contiguous())
    q, k, v, g, beta = (sel(d[n]) for n in ("q", "k", "v", "g", "beta"))
    ref = oracle.bwd(q, k, v, g, beta, offs, d["scale"], sel(do), gate_per_key=w.gate_per_key,
                     use_exp2=w.use_exp2, dht=None if dht is None else np32(dht[:, heads]).astype(np.float64))
    tol = TOL[w.dtype]
    return {n: assert_close(sel(got[n]), ref[n], tol, f"{w.name} {n}") for n in NAMES}


def test_backward_packed_workload_sampled_heads():
    # 20 packed documents, 32768 tokens, 32 heads: the whole backward on the
    # GPU, heads 3 and 20 against the oracle
    w = W.WORKLOADS[2]
    d = W.generate(w, 1002, device=DEV)
    meta = gb.make_meta(d["offsets"], w.T, DEV)
    x = [d[n] for n in ("q", "k", "v", "g", "beta")]
    do = torch.randn(x[2].shape, generator=torch.Generator().manual_seed(31)).to(x[2].dtype).to(DEV)
    _, _, ex = gb.gdn_chunk_fwd(*x, d["scale"], meta=meta, want_h=True)
    got = gb.gdn_chunk_bwd(*x, ex["h"], do, d["scale"], meta=meta, want_dh0=False)
    torch.cuda.synchronize()
    errs = _bwd_sampled(d, got, do, [3, 20], list(d["offsets"]))
    print(f"{w.name} backward (heads 3, 20): " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))


def test_backward_split_workload_sampled_heads():
    # the per-key split workload (2 rows of 65536 tokens, 8 segments each, 8
    # heads, log2 gate c = 0.05) through the split backward, as bench.py
    # times it: gradient summaries, adjoint merge, segment backward; heads 1
    # and 6 of both rows against the oracle's unsplit backward
    w = W.WORKLOADS[3]
    d = W.generate(w, 1003, device=DEV)
    x = [d[n] for n in ("q", "k", "v", "g", "beta")]
    seg = d["seg_offsets"]
    meta = gb.make_meta(gb.segment_offsets(w.B, w.T, seg), w.B * w.T, DEV)
    S_ext, M, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, use_exp2=True, q=d["q"])
    S_init, _ = gb.gdn_state_merge(S_ext, M, None, B=w.B, n_seg=w.n_seg, want_final=False)
    _, _, ex = gb.gdn_chunk_fwd(*x, d["scale"], meta=meta, initial_state=S_init, want_h=True, use_exp2=True)
    do = torch.randn(x[2].shape, generator=torch.Generator().manual_seed(33)).to(x[2].dtype).to(DEV)
    got = gb.split_backward(*x, ex["h"], do, d["scale"], seg=seg, M=M, use_exp2=True)
    torch.cuda.synchronize()
    errs = _bwd_sampled(d, got, do, [1, 6], [0, w.T, 2 * w.T])
    print(f"{w.name} split backward (heads 1, 6): " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))


def test_backward_long_workload_sampled_head():
    # one row of 262144 tokens, 32 heads, with dL/d final state: head 5
    # against the oracle (the reverse state pass runs 4096 chunk steps)
    w = W.WORKLOADS[4]
    d = W.generate(w, 1004, device=DEV)
    x = [d[n] for n in ("q", "k", "v", "g", "beta")]
    gen = torch.Generator().manual_seed(35)
    do = torch.randn(x[2].shape, generator=gen).to(x[2].dtype).to(DEV)
    dht = (torch.randn((1, w.H, 128, 128), generator=gen) * 0.1).to(DEV)
    _, _, ex = gb.gdn_chunk_fwd(*x, d["scale"], want_h=True)
    got = gb.gdn_chunk_bwd(*x, ex["h"], do, d["scale"], dht=dht, want_dh0=False)
    del ex
    torch.cuda.synchronize()
    errs = _bwd_sampled(d, got, do, [5], [0, w.T], dht=dht)
    print(f"{w.name} backward (head 5): " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))
