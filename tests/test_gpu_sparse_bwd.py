"""Sparse top-k backward (attn_bwd_sparse_topk) against the fp64 oracle's gradients.

The GPU forward supplies out and lse; the oracle computes the exact gradients of
the same bf16 inputs. Tolerances as the dense backward (derived there from the
bf16 rounding of P and dS before the MFMAs and one rounding of dq): max |g - g_ref|
<= 2e-2 * max |g_ref| per tensor (floor 0.05 on the scale), 1e-2 for the fp32 sink
gradients. The pool gradient is accumulated in fp32 by atomics, so its last bits vary
between runs; dq does not.
"""
import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_backward import TOL_REL, TOL_SINK, _rel_err
from test_gpu_parity import _np, announce

pytestmark = pytest.mark.gpu


def run(q, kv, idx, dout, sinks, scale):
    q, kv, idx, dout = q.cuda(), kv.cuda(), idx.cuda(), dout.cuda()
    sk = sinks.cuda() if sinks is not None else None
    out, lse = A.sparse_topk(q, kv, idx, d_v=512, scale=scale, sinks=sk)
    dq = torch.full_like(q, float("nan"))
    dkv = torch.full((kv.shape[0], 512), float("nan"), dtype=torch.float32, device="cuda")
    res = A.sparse_backward(q, kv, idx, out, dout, lse, d_v=512, scale=scale, sinks=sk, dq=dq, dkv=dkv)
    torch.cuda.synchronize()
    return res


def make_case(Sq, N, topk, seed, sinks, special=False):
    inp = synth.randn_sparse(Sq, 64, N, 512, topk, seed=seed, sinks=sinks)
    idx = inp["idx"].clone()
    if special and topk >= 4:
        idx[:, 1] = idx[:, 0]          # a duplicated index in every row
        idx[0, 2] = -1                 # a skipped slot
        idx[min(1, Sq - 1), 3] = N + 5  # an index past the pool, skipped
    g = torch.Generator("cpu").manual_seed(2000 + seed)
    dout = torch.randn((Sq, 64, 512), generator=g).to(torch.bfloat16)
    return inp, idx, dout


CASES = [
    # Sq, N, topk, sinks, special
    (3, 300, 64, False, False),
    (5, 300, 100, True, True),        # ragged last block, duplicates and skipped slots
    (17, 1000, 257, True, False),     # several queries per XCD group, ragged
    (1, 64, 64, False, True),         # every pool row named (with a duplicate)
    (9, 50, 32, True, False),         # small pool: many queries add into the same rows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Sq{c[0]}N{c[1]}k{c[2]}{'s' if c[3] else ''}"
                         f"{'x' if c[4] else ''}")
def test_sparse_bwd_cases(case):
    Sq, N, topk, sinks, special = case
    announce(f"sparse bwd {case}")
    inp, idx, dout = make_case(Sq, N, topk, Sq * 7 + topk, sinks, special)
    scale = 1 / math.sqrt(512)
    dq, dkv, ds = run(inp["q"], inp["kv"], idx, dout, inp["sinks"], scale)
    rq, rkv, rs = oracle.sparse_topk_attention_backward(inp["q"], inp["kv"], idx.numpy(), dout, d_v=512,
                                                        scale=scale, sinks=inp["sinks"])
    errs = {"dq": _rel_err(_np(dq), rq), "dkv": _rel_err(_np(dkv), rkv)}
    assert max(errs.values()) <= TOL_REL, f"{case}: {errs}"
    if rs is not None:
        assert _rel_err(_np(ds), rs) <= TOL_SINK


def test_sparse_bwd_no_slots():
    """topk = 0: no key anywhere, so dq = 0 and the pool gradient is 0."""
    announce("sparse bwd topk=0")
    inp = synth.randn_sparse(4, 64, 40, 512, 8, seed=3, sinks=True)
    idx = torch.zeros((4, 0), dtype=torch.int32)
    dout = torch.ones((4, 64, 512), dtype=torch.bfloat16)
    dq, dkv, ds = run(inp["q"], inp["kv"], idx, dout, inp["sinks"], 0.05)
    assert float(dq.float().abs().max()) == 0.0 and float(dkv.abs().max()) == 0.0


def test_sparse_bwd_repeatable():
    """dq is bitwise repeatable; the pool gradient agrees to fp32 summation order."""
    announce("sparse bwd repeat")
    inp, idx, dout = make_case(9, 100, 64, 11, True)
    a = run(inp["q"], inp["kv"], idx, dout, inp["sinks"], 0.04)
    b = run(inp["q"], inp["kv"], idx, dout, inp["sinks"], 0.04)
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert float((a[1] - b[1]).abs().max()) <= 1e-5 * float(a[1].abs().max())


def test_sparse_bwd_rejects():
    q = torch.zeros(2, 64, 256, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(10, 256, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    lse = torch.zeros(2, 64, device="cuda")
    with pytest.raises(A.AttnUnsupported):       # only d = 512 is compiled
        A.sparse_backward(q, kv, idx, q, q, lse, d_v=256, scale=0.1)
    q5 = torch.zeros(2, 64, 512, dtype=torch.bfloat16, device="cuda")
    kv5 = torch.zeros(10, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnInvalidArgument):   # dsinks without sinks
        A.sparse_backward(q5, kv5, idx, q5, q5, lse, scale=0.1, dsinks=torch.zeros(64, device="cuda"))
    torch.cuda.synchronize()


def test_sparse_bwd_full_workload_sampled():
    """The benchmark's launch at full size (13312 queries x 64 heads, top-k 2176 of a
    65536-row pool). The oracle checks dq of sampled queries (it depends on that
    query only) and the pool gradient of sampled rows (from every query that
    names them)."""
    s = synth.spec(5)
    announce(f"sparse bwd full workload {s.name}")
    inp = synth.make(5)
    dout = synth.make_sparse_dout(s)
    dq, dkv, _ = run(inp["q"], inp["kv"], inp["idx"], dout, inp["sinks"], s.scale)
    idx = inp["idx"].numpy()
    for qs in (0, 4321, s.Sq - 1):
        rq, _, _ = oracle.sparse_topk_attention_backward(inp["q"][qs:qs + 1], inp["kv"], idx[qs:qs + 1],
                                                         dout[qs:qs + 1], d_v=s.d_v, scale=s.scale)
        e = _rel_err(_np(dq[qs:qs + 1]), rq)
        assert e <= TOL_REL, f"dq of query {qs}: {e:.3e}"
    for n in (7, 40000):
        users = np.nonzero((idx == n).any(axis=1))[0]
        _, rkv, _ = oracle.sparse_topk_attention_backward(inp["q"][users], inp["kv"], idx[users], dout[users],
                                                          d_v=s.d_v, scale=s.scale)
        e = _rel_err(_np(dkv[n]), rkv[n])
        assert e <= TOL_REL, f"pool row {n} ({len(users)} queries): {e:.3e}"
