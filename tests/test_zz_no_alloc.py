"""The allocation-free split-KV entry point (attn_fwd_dense_splitkv_noalloc).

Its partials go to the library's per-device scratch array instead of a caller
workspace. Through the C ABI it must give what attn_fwd_dense_splitkv gives on
the same arguments (the same kernels over the same key ranges: identical
bits), and both must meet the oracle's bar (max |O - O_ref| <= 2e-2,
max |lse - lse_ref| <= 1e-3). Two calls in a row, the second smaller, show
that the array's leftover contents from one call do not reach the next.
"""
import ctypes
import math

import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_parity import TOL_LSE, TOL_O, _lse_err, _np, _o_err, announce

pytestmark = pytest.mark.gpu


def _outputs(inp):
    B, H, Tq, _ = inp["q"].shape
    dv = inp["v"].shape[-1]
    out = torch.full((B, H, Tq, dv), float("nan"), dtype=inp["q"].dtype, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def _noalloc_call(q, k, v, sk, out, lse, scale, n_splits):
    """The C entry point itself, with the binding's argument struct."""
    lib = A.load_library()
    a = A.dense_args(q, k, v, out, lse, causal=True, scale=scale, sinks=sk)
    st = torch.cuda.current_stream().cuda_stream
    return lib.attn_fwd_dense_splitkv_noalloc(ctypes.byref(a), int(n_splits), ctypes.c_void_p(st))


CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, n_splits: first a large decode, then a smaller one
    (2, 64, 1, 1, 6000, 512, 512, 0),
    (1, 8, 2, 3, 700, 128, 128, 5),
]


def test_noalloc_matches_workspace_call_twice():
    for i, (B, H, Hkv, Tq, Tk, dqk, dv, n) in enumerate(CASES):
        inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=True, seed=4200 + i)
        announce(f"no-alloc split-KV call {i}: B{B} H{H}/{Hkv} {Tq}x{Tk} d{dqk}/{dv} n{n}")
        scale = 1 / math.sqrt(dqk)
        assert 0 < A.splitkv_workspace_bytes(B, H, Hkv, Tq, Tk, dqk, dv, n_splits=n, sinks=True) \
            <= A.NOALLOC_SCRATCH_BYTES
        q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
        sk = inp["sinks"].cuda()
        o_ref, l_ref = _outputs(inp)
        A.dense_splitkv(q, k, v, causal=True, scale=scale, sinks=sk, n_splits=n, out=o_ref, lse=l_ref)
        o_na, l_na = _outputs(inp)
        A.reset_dispatch_counts()
        before = torch.cuda.memory_allocated()
        assert _noalloc_call(q, k, v, sk, o_na, l_na, scale, n) == A.ATTN_OK, A.load_library().attn_last_error()
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert A.dispatch_count("splitkv_merge") == 1
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref), "no-alloc and workspace calls differ"
        ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=scale, causal=True, sinks=inp["sinks"])
        eo, el = _o_err(_np(o_na), ro), _lse_err(_np(l_na), rl)
        announce(f"no-alloc call {i}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE


def test_noalloc_binding_and_plain_path():
    """The binding's wrapper gives the same bits; a plan of one range is the plain kernel."""
    inp = synth.randn_dense(1, 8, 2, 64, 100, 128, 128, dtype="bf16", seed=4300)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o1, l1 = _outputs(inp)
    o2, l2 = _outputs(inp)
    A.reset_dispatch_counts()
    A.dense_splitkv_noalloc(q, k, v, o1, l1, n_splits=1)
    A.dense(q, k, v, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert A.dispatch_count("dense_bf16_d128") == 2 and A.dispatch_count("splitkv_merge") == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_rejects_partials_beyond_the_array():
    """64 sequences x 64 heads over 64 ranges of 512-wide partials need 538 MB: refused
    on the host before any launch, outputs untouched."""
    q = torch.zeros((64, 64, 1, 512), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 1, 4096, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.full((64, 64, 1, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((64, 64, 1), 7.0, device="cuda")
    assert A.splitkv_workspace_bytes(64, 64, 1, 1, 4096, 512, 512, n_splits=64) > A.NOALLOC_SCRATCH_BYTES
    with pytest.raises(A.AttnInvalidArgument, match="scratch array"):
        A.dense_splitkv_noalloc(q, k, k, out, lse, n_splits=64)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
