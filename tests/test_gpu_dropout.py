"""Attention dropout (a caller-drawn keep mask shared by the forward and the
backward) against the fp64 oracle on the same mask.

Tolerances as the dense paths: O within 2e-2 and lse within 1e-3 for the forward;
gradients within 2e-2 of max |g_ref| (1e-2 for dsinks) for the backward.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_backward import TOL_REL, TOL_SINK, _rel_err
from test_gpu_parity import TOL_LSE, TOL_O, _lse_err, _np, _o_err, announce

pytestmark = pytest.mark.gpu

P_DROP = 0.2

CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks, window
    (2, 4, 2, 200, 200, 128, 128, True, False, (-1, -1)),
    (1, 4, 1, 130, 300, 64, 64, False, True, (-1, -1)),
    (1, 4, 4, 150, 150, 192, 128, True, True, (-1, -1)),
    (1, 2, 2, 100, 40, 128, 128, True, False, (-1, -1)),     # Tq > Tk: rows that see no key
    (1, 4, 2, 257, 257, 128, 128, True, False, (50, -1)),    # sliding window
    (1, 8, 2, 150, 190, 256, 256, True, True, (-1, -1)),     # 256-wide heads (dK/dV heads split)
    (2, 4, 1, 97, 97, 256, 256, False, False, (30, 20)),     # 256-wide, window both sides
    (1, 8, 1, 130, 150, 512, 512, True, True, (-1, -1)),     # 512-wide: plain forward, then the dropout pass
    (1, 4, 2, 70, 70, 512, 512, False, False, (25, -1)),     # 512-wide with a window
    (1, 4, 1, 90, 40, 512, 512, True, True, (-1, -1)),       # 512-wide, Tq > Tk: rows that see no key
]


def setup(case, seed):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=seed)
    keep = synth.make_keep(B, H, Tq, Tk, P_DROP, seed=seed)
    return inp, keep, synth.pack_keep(keep).cuda()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[3]}x{c[4]}d{c[5]}{'c' if c[7] else 'n'}"
                         f"{'s' if c[8] else ''}w{c[9][0]}")
def test_dropout_forward(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    announce(f"dropout fwd {case}")
    inp, keep, kw = setup(case, Tq + Tk + dqk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    scale = 1 / math.sqrt(dqk)
    A.reset_dispatch_counts()
    out, lse = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, window=window, keep=kw, p_drop=P_DROP)
    if dqk == 512:  # the mask is applied inside the fused 512-wide kernel, in one launch
        assert A.dispatch_count("dense_bf16_d512_dropout") == 1 and A.dispatch_count("dense_dropout_bf16") == 0
    else:
        assert A.dispatch_count("dense_dropout_bf16") == 1
    plain, _ = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=scale, causal=causal, sinks=inp["sinks"],
                                    window=window, keep=keep.numpy(), p_drop=P_DROP)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"
    # the dropout is applied, not ignored (the defect the TransformerEngine page's review names)
    assert float((out.float() - plain.float()).abs().max()) > 0.05


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[3]}x{c[4]}d{c[5]}{'c' if c[7] else 'n'}"
                         f"{'s' if c[8] else ''}w{c[9][0]}")
def test_dropout_backward(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    announce(f"dropout bwd {case}")
    inp, keep, kw = setup(case, 3 * Tq + Tk + dqk)
    dout = synth.randn_dout(B, H, Tq, dv, seed=Tq + dqk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    scale = 1 / math.sqrt(dqk)
    out, lse = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, window=window, keep=kw, p_drop=P_DROP)
    dq, dk, dv_, ds = A.dense_backward(q, k, v, out, dout.cuda(), lse, causal=causal, scale=scale, sinks=sk,
                                       window=window, keep=kw, p_drop=P_DROP)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.dense_attention_backward(inp["q"], inp["k"], inp["v"], dout, scale=scale, causal=causal,
                                                     sinks=inp["sinks"], window=window, keep=keep.numpy(),
                                                     p_drop=P_DROP)
    errs = {"dq": _rel_err(_np(dq), rq), "dk": _rel_err(_np(dk), rk), "dv": _rel_err(_np(dv_), rv)}
    assert max(errs.values()) <= TOL_REL, f"{case}: {errs}"
    if rs is not None:
        assert _rel_err(_np(ds), rs) <= TOL_SINK


def test_dropout_full_workload_sampled():
    """The gqa workload (B2 H32/8 T4096 d128 causal) with p = 0.1: sampled rows of the
    forward against the oracle on the same mask."""
    s = synth.spec(2)
    announce(f"dropout full workload {s.name}")
    inp = synth.make(2)
    keep = synth.make_keep(s.B, s.H, s.Tq, s.Tk, 0.1, seed=2)
    out, lse = A.dense(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal=True, scale=s.scale,
                       keep=synth.pack_keep(keep).cuda(), p_drop=0.1)
    torch.cuda.synchronize()
    rows = [(0, 0, 0), (1, 31, 4095), (0, 17, 2048), (1, 8, 333)]
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=s.scale, causal=True, rows=rows,
                                    keep=keep.numpy(), p_drop=0.1)
    got_o = torch.stack([out[b, h, t] for b, h, t in rows])
    got_l = torch.stack([lse[b, h, t] for b, h, t in rows])
    eo, el = _o_err(_np(got_o), ro), _lse_err(_np(got_l), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"


def test_dropout_rejects():
    inp = synth.randn_dense(1, 2, 1, 8, 8, 128, 128, dtype="bf16", seed=1)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    kw = synth.pack_keep(synth.make_keep(1, 2, 8, 8, 0.5, seed=1)).cuda()
    with pytest.raises(A.AttnUnsupported):        # dropout is compiled for bf16 inputs only
        A.dense(q.float(), k.float(), v.float(), keep=kw, p_drop=0.5)
    q2, k2 = q, k
    out = torch.empty_like(q2)
    lse = torch.empty((1, 2, 8), device="cuda")
    a = A.dense_args(q2, k2, k2, out, lse, causal=True, scale=0.1, keep=kw, p_drop=0.5)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    lib = A.load_library()
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.attn_fwd_dense_splitkv(ctypes.byref(a), 2, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                    ctypes.c_void_p(st))
    assert rc == A.ATTN_UNSUPPORTED                # split-KV takes no mask
    with pytest.raises(A.AttnInvalidArgument):     # p_drop out of range
        A.dense(q2, k2, k2, keep=kw, p_drop=1.0)
    torch.cuda.synchronize()
