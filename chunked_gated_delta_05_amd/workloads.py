"""Seeded synthetic workloads for the chunked gated delta rule forward.

This module only draws inputs: it holds none of the method's arithmetic, so
both the HIP path and the CPU oracle can be fed from it. The five named
workloads are the shapes the forward is measured and checked on:

  0 gdn_tiny_fp32   B=1, T=512,    H=4,  fp32, scalar gate (ln units)
  1 gdn_dense_bf16  B=4, T=4096,   H=16, bf16, scalar gate, BSND
  2 gdn_varlen_tnd  T=32768 packed (20 documents, lengths in [100, 4000]), H=32, bf16, TND
  3 kda_split       B=2, T=65536,  H=8,  bf16, per-key gate (log2 units), 8 segments of 8192
  4 gdn_long        B=1, T=262144, H=32, bf16, scalar gate, final state on

Distributions (all K = V = 128): q, k ~ N(0, 1) then divided by their L2 norm
per (token, head); v ~ N(0, 1); g = -c * softplus(N(0, 1)) with c = 0.1 (ln
units) or c = 0.05 (log2 units, per key); beta = sigmoid(N(0, 1)); scale =
1/sqrt(128); zero initial state. q, k, v and beta are cast to the workload's
dtype after the fp32 transforms; g stays fp32.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dtype: str = "bf16"          # "bf16" or "fp32": q, k, v, beta and o
    layout: str = "BSND"         # "BSND" [B,T,H,D] or "TND" [T,H,D] (packed, B == 1)
    gate_per_key: bool = False   # g is [.., H] (scalar) or [.., H, K] (per key)
    use_exp2: bool = False       # decay = 2^g (True) or e^g (False)
    gate_coef: float = 0.1       # g = -gate_coef * softplus(N(0, 1))
    n_docs: int = 0              # TND: number of packed documents
    doc_len: tuple = (100, 4000) # TND: document length range
    n_seg: int = 0               # split: segments per batch row
    final_state: bool = False
    K: int = 128
    V: int = 128


WORKLOADS = [
    Workload("gdn_tiny_fp32", B=1, T=512, H=4, dtype="fp32"),
    Workload("gdn_dense_bf16", B=4, T=4096, H=16),
    Workload("gdn_varlen_tnd", B=1, T=32768, H=32, layout="TND", n_docs=20),
    Workload("kda_split", B=2, T=65536, H=8, gate_per_key=True, use_exp2=True,
             gate_coef=0.05, n_seg=8),
    Workload("gdn_long", B=1, T=262144, H=32, final_state=True),
]


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def doc_lengths(n_docs: int, total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Seeded document lengths: uniform draws in [lo, hi], rescaled to sum to
    ``total``, clamped to [lo, hi], the residual spread +-1 cyclically in index
    order (skipping documents at a bound). Redrawn with seed + 1 until at
    least three quarters of the lengths are not multiples of 64."""
    if n_docs < 1 or n_docs * lo > total or n_docs * hi < total:
        raise ValueError(f"{n_docs} documents of {lo}..{hi} tokens cannot sum to {total}")
    for _ in range(1000):
        gen = torch.Generator("cpu").manual_seed(seed)
        raw = torch.randint(lo, hi + 1, (n_docs,), generator=gen).tolist()
        s = sum(raw)
        lens = [min(hi, max(lo, (x * total) // s)) for x in raw]
        resid = total - sum(lens)
        i = 0
        guard = 0
        while resid != 0 and guard < 100 * n_docs:
            step = 1 if resid > 0 else -1
            if lo <= lens[i] + step <= hi:
                lens[i] += step
                resid -= step
            i = (i + 1) % n_docs
            guard += 1
        if resid == 0 and sum(x % 64 != 0 for x in lens) * 4 >= 3 * n_docs:
            return lens
        seed += 1
    raise ValueError(f"no seeded draw of {n_docs} document lengths fits {total} tokens")


def cu_from_lengths(lens) -> list[int]:
    out = [0]
    for x in lens:
        out.append(out[-1] + int(x))
    return out


def _l2n(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def generate(w: Workload, seed: int, device: str | torch.device = "cpu") -> dict:
    """Draw the inputs of workload ``w``. Tensors are created on ``device``
    with a generator seeded by ``seed`` (the draw order is fixed: document
    lengths, q, k, v, g, beta).

    Returns a dict: q, k, v ([B,T,H,K] or [T,H,K]); g; beta; scale; offsets
    (unit token offsets over the flat token axis, or None for dense rows);
    cu_seqlens (TND) and seg_offsets (split, per row) when they apply."""
    dev = torch.device(device)
    cu = None
    if w.layout == "TND":
        lens = doc_lengths(w.n_docs, w.T, w.doc_len[0], w.doc_len[1], seed)
        cu = cu_from_lengths(lens)
    gen = torch.Generator(dev.type).manual_seed(seed)
    lead = (w.T,) if w.layout == "TND" else (w.B, w.T)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    dt = torch_dtype(w.dtype)
    q = _l2n(randn(*lead, w.H, w.K)).to(dt)
    k = _l2n(randn(*lead, w.H, w.K)).to(dt)
    v = randn(*lead, w.H, w.V).to(dt)
    gshape = (*lead, w.H, w.K) if w.gate_per_key else (*lead, w.H)
    g = -w.gate_coef * torch.nn.functional.softplus(randn(*gshape))
    beta = torch.sigmoid(randn(*lead, w.H)).to(dt)
    seg = None
    offsets = cu
    if w.n_seg:
        L = w.T // w.n_seg
        seg = [i * L for i in range(w.n_seg)] + [w.T]
        offsets = [b * w.T + s for b in range(w.B) for s in seg[:-1]] + [w.B * w.T]
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "scale": 1.0 / math.sqrt(w.K),
            "offsets": offsets, "cu_seqlens": cu, "seg_offsets": seg, "workload": w}


def flat(x: torch.Tensor, layout: str) -> torch.Tensor:
    """View a BSND [B,T,H,...] tensor (or a TND [T,H,...] one, unchanged) on
    the flat token axis [N,H,...]."""
    return x.reshape(-1, *x.shape[2:]) if layout == "BSND" else x
