"""Shared helpers of the GPU tests: input conversion for the oracle and the
max-abs / rms tolerance of the forward (max|x - ref| <= tol * rms(ref))."""
from __future__ import annotations

import math

import numpy as np
import torch

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def np32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 copy of a (bf16 or fp32) tensor, on the host."""
    return t.detach().float().cpu().numpy()


def flat_inputs(d: dict):
    """q, k, v, g, beta of a generated workload on the flat token axis, as
    numpy fp32 (the oracle's input form)."""
    w = d["workload"]
    f = (lambda x: x.reshape(-1, *x.shape[2:])) if w.layout == "BSND" else (lambda x: x)
    return tuple(np32(f(d[n])) for n in ("q", "k", "v", "g", "beta"))


def unit_offsets(d: dict) -> list:
    w = d["workload"]
    if d["offsets"] is not None:
        return list(d["offsets"])
    return [b * w.T for b in range(w.B + 1)]


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float((ref ** 2).mean()))
    return float(np.abs(x - ref).max()) / (rms if rms > 0 else 1.0)


def assert_close(x, ref, tol, what=""):
    e = rel_err(x, ref)
    assert e <= tol, f"{what}: max|err|/rms(ref) = {e:.3e} > {tol:.1e}"
    return e
