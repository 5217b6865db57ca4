"""gdn_chunk_fwd_noalloc (the allocation-free forward: the library's own
per-GPU scratch instead of a workspace) against gdn_chunk_fwd on the same
inputs, through the C ABI. The two share every kernel, so the results must be
identical bit for bit. Each case makes two calls in a row, the second with a
smaller input, so the second reuses the scratch the first left behind."""
import pytest
import torch

from chunked_gated_delta_05_amd import binding as gb
from chunked_gated_delta_05_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, T, H, seed, per_key=False, dtype="bf16"):
    w = W.Workload("noalloc", B=B, T=T, H=H, dtype=dtype, gate_per_key=per_key, use_exp2=per_key,
                   gate_coef=0.05 if per_key else 0.1)
    d = W.generate(w, seed)
    return {n: d[n].to(DEV) for n in ("q", "k", "v", "g", "beta")}, d["scale"], per_key


@pytest.mark.parametrize("per_key,dtype", [(False, "bf16"), (True, "bf16"), (False, "fp32")])
def test_noalloc_equals_workspace_forward(per_key, dtype):
    # two calls in a row on one GPU, the second on a smaller input
    for B, T, H, seed in ((3, 700, 5, 101), (1, 130, 2, 103)):
        print(f"noalloc per_key={per_key} {dtype} B={B} T={T} H={H}", flush=True)
        x, scale, pk = _inputs(B, T, H, seed, per_key, dtype)
        S0 = (torch.randn(B, H, 128, 128, generator=torch.Generator().manual_seed(seed)) * 0.3).to(DEV)
        o_ref, f_ref, _ = gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, initial_state=S0,
                                           output_final_state=True, use_exp2=pk)
        o = torch.full_like(o_ref, float("nan"))
        f = torch.full_like(f_ref, float("nan"))
        gb.gdn_chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, out=o, final_out=f,
                                 initial_state=S0, use_exp2=pk)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "o differs from gdn_chunk_fwd"
        assert torch.equal(f, f_ref), "final state differs from gdn_chunk_fwd"


def test_noalloc_packed_and_two_stages():
    # packed documents; then the preparation alone followed by a reusing call,
    # which reads what the previous call on this GPU left in the scratch
    cu = W.cu_from_lengths([30, 200, 64, 9, 333])
    base = W.generate(W.Workload("noalloc", B=1, T=cu[-1], H=3), 107)
    x = {n: base[n][0].contiguous().to(DEV) for n in ("q", "k", "v", "g", "beta")}
    meta = gb.make_meta(cu, cu[-1], DEV)
    o_ref, f_ref, _ = gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], base["scale"], meta=meta,
                                       output_final_state=True)
    o = torch.empty_like(o_ref)
    f = torch.empty_like(f_ref)
    gb.gdn_chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], base["scale"], out=o, final_out=f,
                             meta=meta)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
    o.zero_()
    f.zero_()
    gb.gdn_chunk_fwd_noalloc(x["q"], x["k"], None, x["g"], x["beta"], base["scale"], out=o, meta=meta,
                             flags=gb.FLAG_PREPARE_ONLY)
    gb.gdn_chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], base["scale"], out=o, final_out=f,
                             meta=meta, flags=gb.FLAG_REUSE_PREPARED)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)


def test_noalloc_rejects_problems_beyond_the_scratch():
    # 8192 tokens x 64 heads of bf16 scalar-gate preparation need
    # 128 * 64 * 17 KiB = 136 MiB > 128 MiB: rejected before any launch
    T, H = 8192, 64
    k = torch.zeros(1, T, H, 128, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(1, T, H, device=DEV)
    beta = torch.zeros(1, T, H, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(1, T, H, 128, device=DEV)
    with pytest.raises(ValueError, match="status 4"):
        gb.gdn_chunk_fwd_noalloc(k, k, k, g, beta, out=o)
