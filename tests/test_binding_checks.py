"""The Python binding refuses tensors that do not match each other, before any
launch. The C library receives pointers and sizes only; it cannot see an
allocation's size, so a tensor smaller than the sizes taken from the others, a
dtype that differs from q's, or a host tensor would become an out-of-bounds or
host-pointer access on the device. These run on the CPU: the checks of shapes
and dtypes come before the device check, and a call whose tensors all match
stops at the device check.
"""
import pytest
import torch

import attention_forward_attn_amd as A
import synth

Err = A.AttnInvalidArgument


def dense_inputs(B=1, H=4, Hkv=2, T=16, d=64, dv=64):
    inp = synth.randn_dense(B, H, Hkv, T, T, d, dv, dtype="bf16", sinks=True, seed=1)
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16)
    lse = torch.empty((B, H, T), dtype=torch.float32)
    return inp["q"], inp["k"], inp["v"], out, lse, inp["sinks"]


def call_dense(q, k, v, out, lse, sinks):
    return A.dense(q, k, v, causal=True, sinks=sinks, out=out, lse=lse)


def test_dense_all_matching_stops_at_the_device():
    with pytest.raises(Err, match="must be a GPU tensor"):
        call_dense(*dense_inputs())


@pytest.mark.parametrize("what,match", [
    ("k_dtype", "k must be torch.bfloat16"),
    ("v_dtype", "v must be torch.bfloat16"),
    ("out_dtype", "out must be torch.bfloat16"),
    ("k_width", "k must have shape"),
    ("k_batch", "k must have shape"),
    ("v_heads", "v must have shape"),
    ("v_tokens", "v must have shape"),
    ("out_shape", "out must have shape"),
    ("out_width", "out must have shape"),
    ("lse_shape", "lse must have shape"),
    ("lse_dtype", "lse must be torch.float32"),
    ("lse_strided", "lse must be contiguous"),
    ("sinks_len", "sinks must have shape"),
    ("sinks_dtype", "sinks must be torch.float32"),
    ("q_rank", "q must have shape"),
])
def test_dense_mismatch(what, match):
    q, k, v, out, lse, sinks = dense_inputs()
    if what == "k_dtype":
        k = k.float()
    elif what == "v_dtype":
        v = v.half()
    elif what == "out_dtype":
        out = out.float()
    elif what == "k_width":
        k = k[..., :32]
    elif what == "k_batch":
        k = torch.cat([k, k], 0)
    elif what == "v_heads":
        v = v[:, :1]
    elif what == "v_tokens":
        v = v[:, :, :8]
    elif what == "out_shape":
        out = out[:, :, :8]
    elif what == "out_width":
        out = torch.empty(out.shape[:-1] + (32,), dtype=out.dtype)
    elif what == "lse_shape":
        lse = lse[:, :2]
    elif what == "lse_dtype":
        lse = lse.double()
    elif what == "lse_strided":
        lse = torch.empty((1, 16, 4), dtype=torch.float32).transpose(1, 2)
    elif what == "sinks_len":
        sinks = sinks[:2].contiguous()
    elif what == "sinks_dtype":
        sinks = sinks.double()
    elif what == "q_rank":
        q = q[0]
    with pytest.raises(Err, match=match):
        call_dense(q, k, v, out, lse, sinks)


def test_dense_splitkv_and_extras_check_too():
    q, k, v, out, lse, sinks = dense_inputs()
    with pytest.raises(Err, match="v must have shape"):
        A.dense_splitkv(q, k, v[:, :, :8], out=out, lse=lse, sinks=sinks)
    with pytest.raises(Err, match="out must have shape"):
        A.dense_extras(q, k, v, out[:, :1], lse, sinks=sinks, want_p=False)


def sparse_inputs(Sq=3, Hq=16, N=40, d=512, topk=8):
    inp = synth.randn_sparse(Sq, Hq, N, d, topk, seed=2, sinks=True)
    out = torch.empty((Sq, Hq, d), dtype=torch.bfloat16)
    lse = torch.empty((Sq, Hq), dtype=torch.float32)
    return inp["q"], inp["kv"], inp["idx"], out, lse, inp["sinks"]


def call_sparse(q, kv, idx, out, lse, sinks):
    return A.sparse_topk(q, kv, idx, d_v=512, sinks=sinks, out=out, lse=lse)


def test_sparse_all_matching_stops_at_the_device():
    with pytest.raises(Err, match="must be a GPU tensor"):
        call_sparse(*sparse_inputs())


@pytest.mark.parametrize("what,match", [
    ("idx_rows", "indices must have shape"),
    ("idx_dtype", "indices must be int32"),
    ("kv_narrow", "kv rows hold"),
    ("kv_dtype", "kv must be torch.bfloat16"),
    ("out_shape", "out must have shape"),
    ("lse_shape", "lse must have shape"),
    ("sinks_len", "sinks must have shape"),
    ("sinks_dtype", "sinks must be torch.float32"),
])
def test_sparse_mismatch(what, match):
    q, kv, idx, out, lse, sinks = sparse_inputs()
    if what == "idx_rows":
        idx = idx[:2]
    elif what == "idx_dtype":
        idx = idx.long()
    elif what == "kv_narrow":
        kv = kv[:, :256]
    elif what == "kv_dtype":
        kv = kv.float()
    elif what == "out_shape":
        out = out[:, :8]
    elif what == "lse_shape":
        lse = lse[:2]
    elif what == "sinks_len":
        sinks = sinks[:4].contiguous()
    elif what == "sinks_dtype":
        sinks = sinks.half()
    with pytest.raises(Err, match=match):
        call_sparse(q, kv, idx, out, lse, sinks)


def test_backward_mismatch():
    q, k, v, out, lse, sinks = dense_inputs(d=128, dv=128)
    dout = torch.zeros_like(out)
    with pytest.raises(Err, match="dq must have shape"):
        A.dense_backward(q, k, v, out, dout, lse, sinks=sinks, dq=q[:, :2])
    with pytest.raises(Err, match="dout must have shape"):
        A.dense_backward(q, k, v, out, dout[..., :64], lse, sinks=sinks)
    with pytest.raises(Err, match="must be a GPU tensor"):
        A.dense_backward(q, k, v, out, dout, lse, sinks=sinks)


def test_sparse_backward_mismatch():
    q, kv, idx, out, lse, sinks = sparse_inputs(Hq=64)
    dout = torch.zeros_like(out)
    with pytest.raises(Err, match="dkv must have shape"):
        A.sparse_backward(q, kv, idx, out, dout, lse, sinks=sinks, dkv=torch.zeros(5, 512))
    with pytest.raises(Err, match="must be a GPU tensor"):
        A.sparse_backward(q, kv, idx, out, dout, lse, sinks=sinks)


def test_quantized_and_fp8_mismatch():
    inp = synth.make_quant_kv(1, 4, 2, 2, 64, 128, "q8_0", seed=3)
    with pytest.raises(Err, match="out must have shape"):
        A.dense_qkv(inp["q"], inp["k"], inp["v"], fmt="q8_0", out=torch.empty(1, 4, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(Err, match="must be a GPU tensor"):
        A.dense_qkv(inp["q"], inp["k"], inp["v"], fmt="q8_0")
    f = synth.make_sparse_fp8(2, 64, 50, 512, 8, seed=4)
    with pytest.raises(Err, match="scales must have shape"):
        A.sparse_fp8(f["q"], f["codes"], f["scales"][:, :2], f["idx"])
    with pytest.raises(Err, match="must be a GPU tensor"):
        A.sparse_fp8(f["q"], f["codes"], f["scales"], f["idx"])


def test_varlen_mismatch():
    inp = synth.make_varlen(dict(synth.VARLEN_PREFILL, n_seqs=2, min_len=4, max_len=9))
    q, k, v = inp["q"], inp["k"], inp["v"]
    cu = torch.from_numpy(inp["cu"])
    with pytest.raises(Err, match="k must be torch.bfloat16"):
        A.dense_varlen(q, k.float(), v, cu, cu, 9)
    with pytest.raises(Err, match="must be a GPU tensor"):
        A.dense_varlen(q, k, v, cu, cu, 9)
