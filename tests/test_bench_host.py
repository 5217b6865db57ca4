"""Host-side logic of bench.py (CPU only): the algorithmic byte model, the CPU
baseline's stream sampling, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import bench
from chunked_gated_delta_05_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WL = {w.name: w for w in W.WORKLOADS}


def test_byte_model_dense_per_chunk_head():
    # bf16, fp32 o, full chunks: 45,952 B (prep) and 94,720 B (state) per chunk-head
    w = WL["gdn_dense_bf16"]
    chunk_heads = w.B * (w.T // 64) * w.H
    bm = bench.byte_model(w, w.B * w.T * w.H, chunk_heads, 4)
    assert bm["prep"] == 45952 * chunk_heads
    assert bm["state"] == 94720 * chunk_heads
    # by parts: q, k in, T and P less their zero blocks, two coefficient rows
    assert 45952 == 64 * (2 * 128 * 2 + 4 + 2) + 2 * 3072 * 2 + 2 * 64 * 4
    assert 94720 == 64 * (3 * 128 * 2 + 128 * 4) + 2 * 3072 * 2 + 2 * 64 * 4


def test_byte_model_counts_partial_chunks_by_tokens():
    # per-token terms follow the tokens, per-chunk terms the chunks: a packed
    # batch of ragged documents costs less than the same chunks when full
    w = WL["gdn_varlen_tnd"]
    full = bench.byte_model(w, 10 * 64 * 2, 10 * 2, 4)
    ragged = bench.byte_model(w, (9 * 64 + 1) * 2, 10 * 2, 4)
    per_tok_state = 3 * 128 * 2 + 128 * 4
    assert full["state"] - ragged["state"] == 63 * 2 * per_tok_state


def test_byte_model_fp32_keeps_whole_tiles():
    w = WL["gdn_tiny_fp32"]
    bm = bench.byte_model(w, 64, 1, 4)
    assert bm["state"] == 64 * (3 * 128 * 4 + 128 * 4) + 2 * 64 * 64 * 4 + 4 * 64 * 4


def test_cpu_baseline_samples_whole_streams():
    # a small packed workload: the sample is whole (document, head) streams in
    # order, and its oracle output has one row per sampled token
    w = W.Workload("bench_small", B=1, T=300, H=2, layout="TND", n_docs=3, doc_len=(60, 150))
    d = W.generate(w, 5)
    offsets = list(d["offsets"])
    cb = bench.cpu_baseline(d, w, offsets, budget_s=5.0)
    r, sel = cb.pop("_result"), cb.pop("_sel")
    units = list(zip(offsets[:-1], offsets[1:]))
    assert sel == [(a, b, h) for (a, b) in units for h in range(w.H)][:len(sel)]
    assert r["o"].shape == (sum(b - a for a, b, _ in sel), 1, 128)
    assert np.isfinite(r["o"]).all() and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["kind"] == "oracle"


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_backward_io_bytes_closed_form():
    # dense bf16 workload: q, k, v, dL/do (bf16), beta (bf16), g (fp32) read and
    # dq, dk, dv, dg, dbeta (fp32) written per token-head, h (fp32 K x V) per
    # chunk-head, and the dL/d initial state of every row
    import bench
    from chunked_gated_delta_05_amd import workloads as W
    w = W.WORKLOADS[1]
    th, ch, ns = 4 * 4096 * 16, 4 * 64 * 16, 4 * 16
    per_th = 4 * 128 * 2 + 2 + 4 + 3 * 128 * 4 + 4 + 4
    assert bench.bwd_io_bytes(w, th, ch, ns, False) == th * per_th + ch * 128 * 128 * 4 + ns * 128 * 128 * 4
    wk = W.WORKLOADS[3]                          # per-key gate: g and dg are K-vectors
    per_th_k = 4 * 128 * 2 + 2 + 4 * 128 + 3 * 128 * 4 + 4 * 128 + 4
    assert bench.bwd_io_bytes(wk, 10, 1, 1, True) == 10 * per_th_k + 128 * 128 * 4 + 2 * 128 * 128 * 4
