"""The binding's argument checks (CPU only). The C ABI takes bare pointers
and cannot check buffer sizes, so the binding checks every tensor's dtype,
shape, contiguity and device before the C call. Each mismatch below must
raise ValueError naming the offending argument, before anything touches a
GPU; a consistent call on CPU tensors is rejected last, for not being on
the GPU."""
import pytest
import torch

from chunked_gated_delta_05_amd import binding as gb

B, T, H, K = 2, 70, 3, 128


def inputs(dtype=torch.bfloat16, per_key=False):
    q = torch.zeros(B, T, H, K, dtype=dtype)
    g = torch.zeros(B, T, H, K) if per_key else torch.zeros(B, T, H)
    return {"q": q, "k": q.clone(), "v": q.clone(), "g": g, "beta": torch.zeros(B, T, H, dtype=dtype)}


def call(x, **kw):
    return gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], **kw)


def test_consistent_cpu_call_is_rejected_for_the_device():
    with pytest.raises(ValueError, match="GPU tensors"):
        call(inputs())
    with pytest.raises(ValueError, match="GPU tensors"):
        call(inputs(torch.float32, per_key=True), out=torch.empty(B, T, H, K))


@pytest.mark.parametrize("name,bad,msg", [
    ("q", torch.zeros(B, T, H, K), "q must be torch.bfloat16"),                   # fp32 q with bf16 k
    ("beta", torch.zeros(B, T, H), "beta must be torch.bfloat16"),
    ("v", torch.zeros(B, T, H, K, dtype=torch.float16), "v must be torch.bfloat16"),
    ("g", torch.zeros(B, T, H, dtype=torch.bfloat16), "g must be torch.float32"),
    ("q", torch.zeros(B, T - 1, H, K, dtype=torch.bfloat16), "q must have shape"),
    ("v", torch.zeros(B, T, H, K, 1, dtype=torch.bfloat16), "v must have shape"),
    ("beta", torch.zeros(B, T, H + 1, dtype=torch.bfloat16), "beta must have shape"),
    ("g", torch.zeros(B, T, H + 1), "g must have shape"),
    ("g", torch.zeros(B, T, H, 64), "g must have shape"),
    ("g", torch.zeros(B, T), "g must be"),
    ("q", torch.zeros(B, T, K, H, dtype=torch.bfloat16).transpose(-1, -2), "q must be contiguous"),
])
def test_each_input_mismatch_raises(name, bad, msg):
    x = inputs()
    x[name] = bad
    with pytest.raises(ValueError, match=msg):
        call(x)


@pytest.mark.parametrize("kw,msg", [
    ({"out": torch.zeros(B, T, H, K, dtype=torch.bfloat16)}, "out must be torch.float32"),   # default o_dtype fp32
    ({"out": torch.zeros(B, T, H, K), "o_dtype": torch.bfloat16}, "out must be torch.bfloat16"),
    ({"out": torch.zeros(B, T, H, K - 1)}, "out must have shape"),
    ({"out": torch.zeros(B, T, K, H).transpose(-1, -2)}, "out must be contiguous"),
    ({"final_out": torch.zeros(B, H, K, K, dtype=torch.bfloat16)}, "final_out must be torch.float32"),
    ({"final_out": torch.zeros(B + 1, H, K, K)}, "final_out must have shape"),
    ({"initial_state": torch.zeros(B, H, K, K - 1)}, "initial_state must have shape"),
    ({"initial_state": torch.zeros(B, H, K, K, dtype=torch.float64)}, "initial_state must be torch.float32"),
    ({"o_dtype": torch.float16}, "unsupported output dtype"),
])
def test_each_output_mismatch_raises(kw, msg):
    with pytest.raises(ValueError, match=msg):
        call(inputs(), **kw)


def test_per_key_preparation_needs_q():
    x = inputs(per_key=True)
    with pytest.raises(ValueError, match="needs q"):
        gb.gdn_chunk_fwd(None, x["k"], None, x["g"], x["beta"], flags=gb.FLAG_PREPARE_ONLY)


def test_summary_and_merge_buffers():
    x = inputs()
    meta = gb.UnitMeta([0, 35, 70, 105, 140], None, torch.zeros(5, dtype=torch.int32),
                       torch.zeros(5, dtype=torch.int32), torch.zeros(4, 2, dtype=torch.int32), 4)
    with pytest.raises(ValueError, match="mode must be"):
        gb.gdn_state_summary(x["k"], x["v"], x["g"], x["beta"], meta=meta, mode=3)
    S = torch.zeros(4, H, K, K)
    with pytest.raises(ValueError, match="GPU"):
        gb.gdn_state_merge(S, S, B=2, n_seg=2)
