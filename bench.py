"""Benchmark of the chunked gated delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--workload NAME] [--no-cpu]

The default workload is gdn_dense_bf16 (B=4, T=4096, H=16, bf16); --workload
also takes gdn_tiny_fp32, gdn_varlen_tnd (packed documents), kda_split (per-key
gate; the step is the sequence split: summaries, merge, correction) and
gdn_long.

A step is one full forward (chunk preparation + state pass with the fused
output), one gdn_chunk_fwd call, over one batch of synthetic inputs already
resident in HBM. Untimed steps for --settle seconds (the clocks ramp up over
the first milliseconds of back-to-back work), W untimed warmup steps, then K
timed steps between device synchronisations, with nothing else on the stream;
one JSON line on stdout. Per-kernel durations come from a second pass of K
steps, each run as its two stages (prepare only, then reuse the preparation)
with HIP events recorded on the launch stream before, between and after the
two kernels (two events a step: a step's end event is the next step's start
event); that pass's own time per step is reported beside the first. Back-to-back steps reuse
inputs that partly stay in the 256 MiB last-level cache, so a few more steps
are also timed one by one after a cache-evicting write ("cold"). The CPU
baseline times the fp64 oracle on a bounded sample of the same workload
(host threads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked GDN fwd tokens/s and TFLOP/s at H=16,K=V=128 (bf16); % MFMA roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
FLOP_PER_TOKEN_HEAD = 139264   # 2 [3KV + (BT/2)(3K + 2V)], K = V = 128, BT = 64
# The backward's products per token-head, as the method states them: seven
# full ones of K x V per token (Kg dh', Qd^T dO, Kd^T Z, the recomputed Kd h,
# dO h^T, v_new dh'^T, Z h^T) and eleven triangular ones of (BT/2) x 128 per
# token (P^T dO, Tb^T dvn, the recomputed Tb Y, dP, dTb, K K^T and the four
# dq / dk products with the decayed dL and dP, and the dL solve through T
# counted as one). The work unit of the backward line, whatever regrouping the
# kernels use.
BWD_FLOP_PER_TOKEN_HEAD = 2 * (7 * 128 * 128 + 11 * 32 * 128)
KERNEL_SRC = os.path.join(ROOT, "chunked_gated_delta_05_amd", "csrc", "gdn_kernels.hip")


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel source's code: comments, trailing blanks and
    empty lines removed, so that a comment-only edit keeps the committed
    counter summaries attached while any code change detaches them."""
    import re

    src = open(KERNEL_SRC, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def byte_model(w, token_heads: int, chunk_heads: int, o_bytes: int) -> dict:
    """Algorithmic bytes per launch of the scalar-gate kernels: what each
    kernel must read and write by its contract (every byte once). Per
    token-head (es = input element size) and per chunk-head (a chunk of up to
    64 tokens of one head):
      bf16 inputs (fp16 operands):
        prep : q, k (2*128*2), g (4), beta (2) per token-head;
               T, P (2 * 3072 * 2: the 64 x 64 tiles less the four zero
               16 x 16 blocks that token rows 0..31 never use; beta is
               folded into T) and two per-row coefficient rows (2*64*4) per
               chunk-head
        state: q, k, v (3*128*2), o (128*o_bytes) per token-head; T, P and
               the coefficient rows per chunk-head
      fp32 inputs (fp32 operands): the same with es = 4, whole T and P tiles
        (2*64*64*4) and four gate rows (4*64*4)"""
    es = 2 if w.dtype == "bf16" else 4
    tp = 2 * 3072 * 2 if w.dtype == "bf16" else 2 * 64 * 64 * 4
    coef = 2 * 64 * 4 if w.dtype == "bf16" else 4 * 64 * 4
    prep = token_heads * (2 * 128 * es + 4 + es) + chunk_heads * (tp + coef)
    state = token_heads * (3 * 128 * es + 128 * o_bytes) + chunk_heads * (tp + coef)
    return {"prep": prep, "state": state}


def io_bytes(w, token_heads: int, n_states: int, o_bytes: int) -> int:
    """The method's algorithmic bytes per forward: every input read once and
    every output written once - q, k, v (128 elements each), beta (one), the
    gate (one fp32 word, or 128 per key) per token-head, o (128 elements of
    o_bytes) per token-head, and the fp32 128 x 128 final state of each
    (unit, head) when it is an output. Nothing the implementation chooses to
    keep in between (workspace tiles, coefficient rows) counts."""
    es = 2 if w.dtype == "bf16" else 4
    per_th = 3 * 128 * es + es + 4 * (128 if w.gate_per_key else 1) + 128 * o_bytes
    return per_th * token_heads + (n_states * 128 * 128 * 4 if w.final_state else 0)


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on another version of the kernels."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(d, w, offsets, budget_s: float = 15.0) -> dict:
    """The fp64 oracle on a bounded sample of the workload's (unit, head)
    streams, on this host's cores: whole streams, in (unit, head) order, as
    many as fit the budget (estimated from one stream's first tokens on one
    thread). Every selected stream becomes one single-head unit of a packed
    oracle input."""
    import numpy as np

    import oracle

    threads = max(1, len(os.sched_getaffinity(0)))
    flat = {n: W_flat(d[n], w.layout) for n in ("q", "k", "v", "g", "beta")}
    units = list(zip(offsets[:-1], offsets[1:]))
    streams = [(a, b, h) for (a, b) in units for h in range(w.H)]

    def pack(sel, limit=None):
        cut = [(a, b if limit is None else min(b, a + limit), h) for a, b, h in sel]
        arrs = {n: np.ascontiguousarray(np.concatenate(
            [flat[n][a:b, h:h + 1].float().cpu().numpy() for a, b, h in cut], axis=0))
            for n in flat}
        offs = [0]
        for a, b, _ in cut:
            offs.append(offs[-1] + (b - a))
        return arrs, offs

    def run(sel, nthr, limit=None):
        x, offs = pack(sel, limit)
        t0 = time.perf_counter()
        r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], offs, d["scale"],
                       gate_per_key=w.gate_per_key, use_exp2=w.use_exp2, want_final=False,
                       threads=nthr)
        return time.perf_counter() - t0, r, offs[-1]

    probe = min(2048, streams[0][1] - streams[0][0])
    t1, _, n1 = run(streams[:1], 1, probe)                 # seconds per token, one thread
    per_tok = t1 / max(n1, 1)
    sel, tok = [], 0
    for st in streams:
        L = st[1] - st[0]
        if sel and per_tok * (tok + L) / min(threads, len(sel) + 1) > budget_s:
            break
        sel.append(st)
        tok += L
    used = min(threads, len(sel))
    t, r, token_heads = run(sel, used)
    return {"value": token_heads / w.H / t, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{len(sel)} of {len(streams)} (unit, head) streams of {w.name}, whole streams "
                      f"({token_heads} token-heads), fp64 token recurrence, {t:.1f} s wall on {used} threads",
            "seconds": t, "_result": r, "_sel": sel}


def bwd_io_bytes(w, token_heads: int, chunk_heads: int, n_states: int, with_dht: bool) -> int:
    """The backward's algorithmic bytes: the forward's inputs q, k, v, beta,
    g and dL/do read once per token-head, the fp32 chunk entry states h
    (K x V per chunk-head) and dL/d final state when given, and the fp32
    gradients dq, dk, dv, dg (g's shape), dbeta and dL/d initial state
    written once."""
    es = 2 if w.dtype == "bf16" else 4
    gk = 128 if w.gate_per_key else 1
    reads = token_heads * (4 * 128 * es + es + 4 * gk) + chunk_heads * 128 * 128 * 4
    writes = token_heads * (3 * 128 * 4 + 4 * gk + 4) + n_states * 128 * 128 * 4
    return reads + writes + (n_states * 128 * 128 * 4 if with_dht else 0)


def bench_backward(args, wl, d, gb, W, torch):
    """Times the backward of the workload's forward as a training step runs
    it: gdn_chunk_bwd over the rows or documents (the preparation, the
    reverse state pass, the per-chunk gradients), or for a sequence split the
    split backward (gradient summaries, adjoint merge, every segment's
    backward). The forward that supplies h (and, split, the maps M) runs once,
    untimed. Prints one JSON line."""
    dev = torch.device("cuda:0")
    q, k, v, g, beta = (d[n] for n in ("q", "k", "v", "g", "beta"))
    H, e2 = wl.H, wl.use_exp2
    gen = torch.Generator().manual_seed(2000)
    do = torch.randn(v.shape, generator=gen).to(v.dtype).to(dev)
    tokens = wl.B * wl.T
    offsets = list(d["offsets"]) if wl.layout == "TND" else [b * wl.T for b in range(wl.B + 1)]
    chunks = sum((b - a + 63) // 64 for a, b in zip(offsets[:-1], offsets[1:]))
    n_states = len(offsets) - 1
    dht = (torch.randn((n_states, H, 128, 128), generator=gen) * 0.1).to(dev) if wl.final_state else None
    if wl.n_seg:
        seg = d["seg_offsets"]
        meta = gb.make_meta(gb.segment_offsets(wl.B, wl.T, seg), tokens, dev)
        S_ext, M, _ = gb.gdn_state_summary(k, v, g, beta, meta=meta, use_exp2=e2, q=q)
        S_init, _ = gb.gdn_state_merge(S_ext, M, None, B=wl.B, n_seg=wl.n_seg, want_final=False)
        _, _, ex = gb.gdn_chunk_fwd(q, k, v, g, beta, d["scale"], meta=meta, initial_state=S_init, want_h=True,
                                    use_exp2=e2)
        chunks_run = meta.n_chunks

        def step():
            return gb.split_backward(q, k, v, g, beta, ex["h"], do, d["scale"], seg=seg, M=M, use_exp2=e2)
        path = "gradient summaries + adjoint merge + segment backward"
    else:
        meta = gb.make_meta(d["offsets"], wl.T, dev) if wl.layout == "TND" else None
        _, _, ex = gb.gdn_chunk_fwd(q, k, v, g, beta, d["scale"], meta=meta, want_h=True, use_exp2=e2)
        chunks_run = chunks

        def step():
            return gb.gdn_chunk_bwd(q, k, v, g, beta, ex["h"], do, d["scale"], meta=meta, dht=dht, use_exp2=e2,
                                    want_dh0=False)
        path = "gdn_chunk_bwd"
    for _ in range(max(args.warmup, 1)):
        res = step()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 20))
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    token_heads, chunk_heads = tokens * H, chunks_run * H
    flops = BWD_FLOP_PER_TOKEN_HEAD * token_heads
    io = bwd_io_bytes(wl, token_heads, chunk_heads, n_states, dht is not None)
    tf = flops / (ms * 1e-3) / 1e12
    # bf16 inputs with a scalar gate: fp16 operands (the fp16 MFMA peak, that
    # of bf16); fp32 inputs and the per-key gate: fp32 operands
    h16 = wl.dtype == "bf16" and not wl.gate_per_key
    peak = PEAK_BF16_TFLOPS if h16 else PEAK_FP32_TFLOPS
    out = {"metric": "backward tokens/s", "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": max(args.warmup, 1), "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16" if h16 else "f32",
           "data": "synthetic", "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": H,
                                           "gate": "per_key" if wl.gate_per_key else "scalar",
                                           "input_dtype": wl.dtype, "path": path},
           "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                        "frac": tf / peak, "traffic": None,
                        "note": "whole backward on the method's flop count; " +
                                ("fp16 operands, fp32 accumulation (fp16 MFMA peak)" if h16 else
                                 "fp32 operands (fp32 MFMA peak)")},
           "hbm_frac_io": io / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), "io_bytes": io,
           "flop_per_token_head": BWD_FLOP_PER_TOKEN_HEAD, "cpu_baseline": None}
    print(f"[bench] {wl.name} backward: {ms:.3f} ms/step, {tf:.1f} TFLOP/s ({'fp16' if h16 else 'fp32'} operands)",
          file=sys.stderr, flush=True)
    if not args.no_cpu:
        out["cpu_baseline"], out["parity_sample_err_over_rms"] = bwd_cpu_baseline(d, wl, offsets, do, dht, res)
    print(json.dumps(out), flush=True)


def bwd_cpu_baseline(d, w, offsets, do, dht, res, budget_s: float = 15.0):
    """The fp64 backward oracle on a bounded sample of (unit, head) streams,
    whole streams in order while a one-thread estimate (from one stream's
    first tokens) fits the budget; returns the baseline and the largest
    deviation of the GPU's gradients on those streams over their rms."""
    import numpy as np

    import oracle

    threads = max(1, len(os.sched_getaffinity(0)))
    flat = {n: W_flat(x, w.layout) for n, x in (("q", d["q"]), ("k", d["k"]), ("v", d["v"]), ("g", d["g"]),
                                              ("beta", d["beta"]), ("do", do))}
    streams = [(a, b, h) for a, b in zip(offsets[:-1], offsets[1:]) for h in range(w.H)]

    def pack(sel, limit=None):
        cut = [(a, b if limit is None else min(b, a + limit), h) for a, b, h in sel]
        arrs = {n: np.ascontiguousarray(np.concatenate([flat[n][a:b, h:h + 1].float().cpu().numpy()
                                                        for a, b, h in cut], axis=0)) for n in flat}
        offs = [0]
        for a, b, _ in cut:
            offs.append(offs[-1] + (b - a))
        return arrs, offs

    def run(sel, nthr, limit=None, dh=None):
        x, offs = pack(sel, limit)
        t0 = time.perf_counter()
        r = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], offs, d["scale"], x["do"],
                       gate_per_key=w.gate_per_key, use_exp2=w.use_exp2, dht=dh, threads=nthr)
        return time.perf_counter() - t0, r, offs[-1]

    probe = min(1024, streams[0][1] - streams[0][0])
    t1, _, n1 = run(streams[:1], 1, probe)
    per_tok = t1 / max(n1, 1)
    sel, tok = [], 0
    for st in streams:
        L = st[1] - st[0]
        if sel and per_tok * (tok + L) / min(threads, len(sel) + 1) > budget_s:
            break
        sel.append(st)
        tok += L
    used = min(threads, len(sel))
    dh = None
    if dht is not None:
        units = [offsets.index(a) for a, _, _ in sel]
        dh = np.ascontiguousarray(np.stack([dht[u, h:h + 1].cpu().numpy() for u, (_, _, h) in zip(units, sel)]))
    t, r, token_heads = run(sel, used, dh=dh)
    worst = 0.0
    for name in ("dq", "dk", "dv", "dbeta"):
        got = np.concatenate([W_flat(res[name], w.layout)[a:b, h].float().cpu().numpy() for a, b, h in sel], axis=0)
        ref = r[name][:, 0]
        worst = max(worst, float(np.abs(got - ref).max() / np.sqrt((ref ** 2).mean())))
    cb = {"value": token_heads / w.H / t, "unit": "tokens/s", "cores": used, "kind": "oracle",
          "sample": f"{len(sel)} of {len(streams)} (unit, head) streams of {w.name}, whole streams "
                    f"({token_heads} token-heads), fp64 reverse-mode token recurrence, {t:.1f} s wall on {used} threads",
          "seconds": t}
    return cb, worst


def W_flat(x, layout):
    return x.reshape(-1, *x.shape[2:]) if layout == "BSND" else x


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps, so that the clocks settle")
    ap.add_argument("--workload", default="gdn_dense_bf16",
                    help="gdn_dense_bf16 (default), gdn_tiny_fp32, gdn_varlen_tnd, kda_split, gdn_long")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--o-dtype", choices=("fp32", "input"), default="fp32",
                    help="output dtype: fp32 (default; rounding o to bf16 alone exceeds the "
                         "2e-2 rms parity bar at this workload) or the input dtype")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps timed one by one after a 512 MiB write that evicts the "
                         "last-level cache (reported as cold_ms_per_step; 0 skips)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the workload instead (its own JSON line; at most 20 steps)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device (calibrates the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards by (unit, head) with no communication; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}), flush=True)
        return

    from chunked_gated_delta_05_amd import binding as gb
    from chunked_gated_delta_05_amd import workloads as W

    names = [w.name for w in W.WORKLOADS]
    if args.workload not in names:
        raise SystemExit(f"unknown workload {args.workload}; one of {names}")
    wl = W.WORKLOADS[names.index(args.workload)]
    dev = torch.device("cuda:0")
    d = W.generate(wl, 1000 + names.index(wl.name), device=dev)
    if args.backward:
        bench_backward(args, wl, d, gb, W, torch)
        return
    q, k, v, g, beta = (d[n] for n in ("q", "k", "v", "g", "beta"))
    H, split = wl.H, bool(wl.n_seg)
    o_dtype = torch.float32 if args.o_dtype == "fp32" else v.dtype
    o = torch.empty(v.shape, dtype=o_dtype, device=dev)
    tokens = wl.B * wl.T
    # units of the whole forward (rows or packed documents); the oracle and the
    # byte model count chunks per unit
    offsets = list(d["offsets"]) if wl.layout == "TND" else [b * wl.T for b in range(wl.B + 1)]
    chunks = sum((b - a + 63) // 64 for a, b in zip(offsets[:-1], offsets[1:]))
    meta = gb.make_meta(d["offsets"], wl.T, dev) if wl.layout == "TND" else None
    plan = None
    if split:
        seg = d["seg_offsets"]
        meta = gb.make_meta(gb.segment_offsets(wl.B, wl.T, seg), tokens, dev)
        plan = gb.split_plan_rows(q, k, v, g, beta, d["scale"], seg=seg, use_exp2=wl.use_exp2, o_dtype=o_dtype)
        o = plan.o
    n_units = len(offsets) - 1 if not split else wl.B * wl.n_seg
    fin = torch.empty((n_units, H, 128, 128), dtype=torch.float32, device=dev) if wl.final_state else None
    nb = gb.workspace_bytes(gb._desc(k, H, k.dtype, o_dtype, wl.gate_per_key, wl.use_exp2, d["scale"], meta))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    # unsplit forward: the arguments marshalled once, so that a step costs the
    # host one C call and the GPU never waits for the host
    call = None if split else gb.FwdCall(q, k, v, g, beta, d["scale"], out=o, workspace=ws, meta=meta,
                                         final_out=fin, use_exp2=wl.use_exp2)

    def fwd(ev=None):
        # the whole forward as a caller runs it; ev: events between its launches
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if not split:
            call(0)
            rec(1)
            return
        # sequence split: the summaries that something consumes (none for a
        # row's last segment, S_ext only for its first), the merge, then the
        # forward of every segment from its true entry state (the correction),
        # which also gives the final states
        plan(q, k, v, g, beta, rec=lambda i: rec(i + 1))

    def stages(ev=None):
        # the unsplit forward as its two stages, for the per-kernel events:
        # ev[0] before the preparation, ev[1] between the two kernels; the
        # state pass ends at the next step's ev[0]
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        call(gb.FLAG_PREPARE_ONLY)
        rec(1)
        call(gb.FLAG_REUSE_PREPARED)

    # untimed steps until the clocks have settled (the first ~10-20 ms of
    # back-to-back work run at lower clocks), then the W warmup steps
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            fwd()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # second pass with HIP events on the launch stream: the per-kernel split.
    # Unsplit: the two stages; split: summary (with the preparation), merge,
    # correction. Every boundary is recorded once: a step's end is the next
    # step's start event (each record costs the stream a few microseconds).
    n_ev = 4 if split else 2
    run = fwd if split else stages
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    last = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        run(evs[i])
    last.record()
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    ends = [evs[i + 1][0] for i in range(args.steps - 1)] + [last]
    seg_ms = []
    for j in range(n_ev):
        nxt = (lambda i: evs[i][j + 1]) if j + 1 < n_ev else (lambda i: ends[i])
        seg_ms.append(sum(evs[i][j].elapsed_time(nxt(i)) for i in range(args.steps)) / args.steps)
    names_ms = (["summary_with_prep", "merge", "correction"] if split else ["prep_kernel", "state_kernel"])
    kernel_ms = dict(zip(names_ms, seg_ms[:len(names_ms)]))

    cold = None
    if args.cold_steps > 0:
        # each step after a 512 MiB write (outside the events) that pushes the
        # inputs out of the 256 MiB last-level cache
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cts = []
        for i in range(args.cold_steps):
            flush.fill_(i & 255)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
            run(ev)
            ev[-1].record()
            torch.cuda.synchronize()
            cts.append([ev[0].elapsed_time(ev[-1])] + [ev[j].elapsed_time(ev[j + 1]) for j in range(n_ev)])
        del flush
        cts.sort()
        med = cts[len(cts) // 2]
        cold = {"ms_per_step": med[0], "tokens_per_s": tokens / (med[0] * 1e-3), "steps": args.cold_steps,
                "note": "median of steps timed one by one after a 512 MiB write evicting the cache"}
        cold.update({f"{n}_ms": x for n, x in zip(names_ms, med[1:])})

    token_heads = tokens * H
    chunk_heads = chunks * H
    flops = FLOP_PER_TOKEN_HEAD * token_heads
    tflops = flops / (ms_step * 1e-3) / 1e12
    n_states = (len(offsets) - 1 if not split else wl.B) * H
    io_min = io_bytes(wl, token_heads, n_states, 2 if wl.dtype == "bf16" else 4)   # o at the input precision
    io_call = io_bytes(wl, token_heads, n_states, o.element_size())                # o as this call writes it
    peak_mfma = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    out = {
        "metric": METRIC, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": ms_step,
        "higher_is_better": True, "ms_per_step_event_pass": wall_ev * 1e3 / args.steps,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": H, "K": 128, "V": 128, "chunk": 64,
                   "layout": wl.layout, "gate": "per_key" if wl.gate_per_key else "scalar",
                   "decay_base": 2 if wl.use_exp2 else "e", "o_dtype": str(o_dtype).replace("torch.", ""),
                   "final_state": wl.final_state,
                   **({"documents": len(offsets) - 1} if wl.layout == "TND" else {}),
                   **({"segments_per_row": wl.n_seg, "path": "summary + merge + correction"} if split else {})},
        "tflops": tflops, "mfma_frac": tflops / peak_mfma,
        "io_bytes": io_min, "io_bytes_as_called": io_call,
        "hbm_frac_io": io_min / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "hbm_frac_io_as_called": io_call / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "kernel_ms": kernel_ms,
        "cold": cold,
    }
    # Roofline of the dominant kernel on the method's bytes: the whole
    # forward's I/O (o counted at the input precision) over that kernel's
    # mean event duration. The implementation's own traffic (workspace tiles
    # and coefficient rows, byte_model) is reported beside it as traffic,
    # never as work.
    dom = max(kernel_ms, key=kernel_ms.get)
    dom_ms = kernel_ms[dom]
    achieved = io_min / (dom_ms * 1e-3) / 1e9
    out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                       "traffic": load_traffic(dom, wl.name),
                       "algorithmic_bytes_per_launch": io_min,
                       "algorithmic_bytes_note": "the forward's I/O with o at the input precision; "
                                                 f"{io_call} B with o as written ({out['config']['o_dtype']})",
                       "frac_whole_forward": out["hbm_frac_io"]}
    if cold is not None:
        out["roofline"]["frac_cold"] = io_min / (cold[f"{dom}_ms"] * 1e-3) / (PEAK_HBM_GBS * 1e9)
        out["roofline"]["frac_whole_forward_cold"] = io_min / (cold["ms_per_step"] * 1e-3) / (PEAK_HBM_GBS * 1e9)
    if not wl.gate_per_key:
        bm = byte_model(wl, token_heads, chunk_heads, o.element_size())
        out["implementation_traffic_bytes"] = {"prep_kernel": bm["prep"], "state_kernel": bm["state"],
                                               "note": "what each kernel reads and writes, workspace included"}
    print(f"[bench] {wl.name}: {ms_step:.4f} ms/step, "
          + ", ".join(f"{n} {x:.4f} ms" for n, x in kernel_ms.items()) + f", {tflops:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    if not args.no_cpu:
        import numpy as np

        cb = cpu_baseline(d, wl, offsets)
        r, sel = cb.pop("_result"), cb.pop("_sel")
        of = W_flat(o, wl.layout)
        got = np.concatenate([of[a:b, h].float().cpu().numpy() for a, b, h in sel], axis=0)
        ref = r["o"][:, 0]
        out["parity_sample_err_over_rms"] = float(np.abs(got - ref).max() / np.sqrt((ref ** 2).mean()))
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
