"""Packed documents split into segments (the packed context-parallel plan of
the Diff Coverage page, on one GPU): pieces from gdn_split_meta, summaries of
the selected pieces only, the piece merge and the correction forward,
against the fp64 oracle and against the unsplit packed forward.

Tolerances as in the forward parity tests: max |x - oracle| <= tol * rms
with tol = 1e-4 (fp32 inputs) and 2e-2 (bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_05_amd import binding as gb
from chunked_gated_delta_05_amd import workloads as W
from oracle import varlen
from tests.gpu_helpers import TOL, assert_close, np32, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _packed(lens, H, dtype, per_key, seed):
    total = sum(lens)
    w = W.Workload("packed", B=1, T=total, H=H, dtype=dtype, layout="TND", gate_per_key=per_key,
                   use_exp2=per_key, gate_coef=0.02 if per_key else 0.05, n_docs=len(lens))
    d = W.generate(w, seed)
    d["offsets"] = W.cu_from_lengths(lens)
    for n in ("q", "k", "v", "g", "beta"):
        d[n] = d[n].to(DEV)
    return w, d


def _np(d):
    return tuple(np32(d[n]) for n in ("q", "k", "v", "g", "beta"))


# documents of 70, 300 (spans three segments), 5 (inside one), 64 and 161
# tokens; segment cuts on a document boundary (70 is not one), one token into
# a document, and inside chunks
LENS = [70, 300, 5, 64, 161]
SEGS = [[0, 150, 300, 375, 600], [0, 71, 200, 439, 600], [0, 600]]


@pytest.mark.parametrize("segs", SEGS)
@pytest.mark.parametrize("per_key,dtype,with_s0,ext_only", [(False, "bf16", False, True), (False, "fp32", True, False),
                                                            (True, "bf16", True, False), (True, "fp32", False, True),
                                                            (True, "bf16", False, False)])
def test_packed_split_matches_oracle(segs, per_key, dtype, with_s0, ext_only):
    # ext_only: the summaries of pieces that enter from zero in a launch of
    # their own, S_ext only (their maps are never computed)
    print(f"packed split per_key={per_key} {dtype} s0={with_s0} ext_only={ext_only} segs={segs}", flush=True)
    w, d = _packed(LENS, 2, dtype, per_key, 401 + len(segs))
    docs = d["offsets"]
    n_docs = len(docs) - 1
    S0 = None
    if with_s0:
        S0 = (torch.randn(n_docs, 2, 128, 128, generator=torch.Generator().manual_seed(5)) * 0.3).to(DEV)
    o, fin, S_in = gb.split_forward_packed(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                           doc_offsets=docs, seg_offsets=segs, use_exp2=w.use_exp2,
                                           initial_state=S0, ext_only_launch=ext_only)
    torch.cuda.synchronize()
    q, k, v, g, beta = _np(d)
    s0 = None if S0 is None else np32(S0).astype(np.float64)
    r = oracle.fwd(q, k, v, g, beta, docs, d["scale"], gate_per_key=per_key, use_exp2=w.use_exp2, S0=s0)
    tol = TOL[dtype]
    assert_close(np32(o), r["o"], tol, "split o")
    assert_close(np32(fin), r["final"], tol, "document final states")
    # entry states of the pieces against the oracle's summaries and merge
    pieces, pdoc, _ = varlen.split_pieces(docs, segs)
    s = oracle.summary(k, v, g, beta, pieces, gate_per_key=per_key, use_exp2=w.use_exp2)
    want = oracle.merge_pieces(s["S_ext"], s["M"], pdoc, s0)
    assert_close(np32(S_in), want, tol, "piece entry states")
    # and the unsplit packed forward on the GPU
    meta = gb.make_meta(docs, w.T, DEV)
    o_u, f_u, _ = gb.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], meta=meta,
                                   initial_state=S0, output_final_state=True, use_exp2=w.use_exp2)
    torch.cuda.synchronize()
    assert_close(np32(o), np32(o_u), tol, "split vs unsplit o")
    if segs == [0, 600]:
        # no segment cuts: the pieces are the documents, nothing is summarised
        # and the correction pass is the packed forward itself
        assert torch.equal(o, o_u) and torch.equal(fin, f_u)


@pytest.mark.parametrize("ext_only", [False, True])
def test_row_split_plans(ext_only):
    # BSND rows cut into segments, from zero entry states: the first segment
    # of each row needs S_ext only, the last no summary at all
    print(f"row split ext_only={ext_only}", flush=True)
    w = W.Workload("rows", B=2, T=300, H=2, dtype="bf16", gate_per_key=True, use_exp2=True, gate_coef=0.02)
    d = W.generate(w, 441)
    for n in ("q", "k", "v", "g", "beta"):
        d[n] = d[n].to(DEV)
    seg = [0, 64, 100, 230, 300]
    o, fin, S_in = gb.split_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], seg=seg,
                                    use_exp2=True, ext_only_launch=ext_only)
    torch.cuda.synchronize()
    flat = lambda x: np32(x.reshape(-1, *x.shape[2:]))
    r = oracle.fwd(*(flat(d[n]) for n in ("q", "k", "v", "g", "beta")), [0, 300, 600], d["scale"],
                   gate_per_key=True, use_exp2=True)
    assert_close(flat(o), r["o"], TOL["bf16"], "row split o")
    assert_close(np32(fin), r["final"], TOL["bf16"], "row split final")
    assert bool((S_in[0] == 0).all()) and bool((S_in[4] == 0).all())


def test_summary_selection_writes_only_selected_slots():
    # listed units get exactly the full-run summary; the others keep what the
    # caller left there
    print("summary selection", flush=True)
    w, d = _packed(LENS, 2, "bf16", False, 431)
    pieces = [0, 70, 150, 300, 370, 375, 439, 600]
    meta = gb.make_meta(pieces, w.T, DEV)
    e_all, m_all, _ = gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, mode=0)
    sel = [5, 1, 3]
    sentinel = 12345.0
    e_sel = torch.full_like(e_all, sentinel)
    m_sel = torch.full_like(m_all, sentinel)
    units = torch.tensor(sel, dtype=torch.int32, device=DEV)
    gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, mode=0, S_ext=e_sel, M=m_sel,
                         units=units)
    # an empty selection runs the preparation only
    gb.gdn_state_summary(d["k"], d["v"], d["g"], d["beta"], meta=meta, mode=0, S_ext=e_sel, M=m_sel,
                         units=units[:0])
    torch.cuda.synchronize()
    for u in range(len(pieces) - 1):
        if u in sel:
            assert torch.equal(e_sel[u], e_all[u]) and torch.equal(m_sel[u], m_all[u]), f"unit {u}"
        else:
            assert bool((e_sel[u] == sentinel).all()) and bool((m_sel[u] == sentinel).all()), f"unit {u}"


@pytest.mark.parametrize("with_s0", [False, True])
def test_merge_pieces_kernel_against_oracle(with_s0):
    # random summaries: pieces 0-1-2 of document 0, 3 alone, 4-5 of document
    # 2; without entry states the maps of pieces 0 and 4 are never read, so
    # they hold NaN here and must not reach the result
    print(f"piece merge s0={with_s0}", flush=True)
    H = 3
    gen = torch.Generator().manual_seed(17)
    pdoc = [0, 0, 0, 1, 2, 2]
    n = len(pdoc)
    S_ext = torch.randn(n, H, 128, 128, generator=gen)
    M = torch.randn(n, H, 128, 128, generator=gen) * 0.05
    S0 = torch.randn(3, H, 128, 128, generator=gen) if with_s0 else None
    want = oracle.merge_pieces(S_ext.numpy(), M.numpy(), pdoc, None if S0 is None else S0.numpy())
    Mg = M.clone()
    if not with_s0:
        Mg[0] = float("nan")
        Mg[4] = float("nan")
    S_in = gb.gdn_state_merge_pieces(S_ext.to(DEV), Mg.to(DEV), torch.tensor(pdoc, dtype=torch.int32, device=DEV),
                                     n_docs=3, S0_docs=None if S0 is None else S0.to(DEV))
    torch.cuda.synchronize()
    got = np32(S_in)
    assert np.isfinite(got).all()
    assert_close(got, want, 1e-5, "S_in")
    # pieces that start a document enter exactly with its state
    for p in (0, 3, 4):
        ref = np.zeros((H, 128, 128)) if S0 is None else S0[pdoc[p]].numpy()
        assert np.array_equal(got[p], ref)


def test_workload_varlen_split_full():
    # the packed workload (20 documents, 32768 tokens, 32 heads) cut into 8
    # equal segments: split == unsplit on the GPU, and the oracle on sampled
    # heads
    w = W.WORKLOADS[2]
    d = W.generate(w, 1005, device=DEV)
    docs = list(d["offsets"])
    segs = [i * (w.T // 8) for i in range(8)] + [w.T]
    o, fin, _ = gb.split_forward_packed(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"],
                                        doc_offsets=docs, seg_offsets=segs)
    meta = gb.make_meta(docs, w.T, DEV)
    o_u, f_u, _ = gb.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], meta=meta,
                                   output_final_state=True)
    torch.cuda.synchronize()
    assert_close(np32(o), np32(o_u), TOL["bf16"], "split vs unsplit o")
    assert_close(np32(fin), np32(f_u), TOL["bf16"], "split vs unsplit final")
    heads = [4, 27]
    pick = lambda x: np32(x[:, heads].contiguous())
    r = oracle.fwd(*(pick(d[n]) for n in ("q", "k", "v", "g", "beta")), docs, d["scale"])
    e = assert_close(pick(o), r["o"], TOL["bf16"], "split o (sampled heads)")
    assert_close(np32(fin[:, heads]), r["final"], TOL["bf16"], "split final (sampled heads)")
    print(f"varlen split: sampled o err/rms {e:.2e}")
