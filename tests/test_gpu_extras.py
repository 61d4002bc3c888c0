"""The forward's extra returns (attn_fwd_dense_extras: probabilities and row maxima)
against the fp64 oracle.

The kernel recomputes S in fp32 from the bf16 inputs (relative error ~1e-6) and
takes lse from the GPU forward (|lse - lse_ref| <= 1e-3 by that path's bar), so
|p - p_ref| <= p * (|dS| + |dlse|) stays below 2e-3; row maxima are fp32 sums of
exact bf16 products: within 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_parity import _lse_err, _np, announce

pytestmark = pytest.mark.gpu

TOL_P = 2e-3
TOL_MAX = 1e-4

CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks, window
    (1, 4, 2, 200, 200, 128, 128, True, False, (-1, -1)),
    (2, 2, 1, 150, 300, 64, 64, False, True, (-1, -1)),
    (1, 4, 4, 130, 130, 192, 128, True, True, (40, -1)),
    (1, 2, 1, 97, 33, 256, 256, True, False, (-1, -1)),     # Tq > Tk: rows that see no key
    (1, 8, 1, 70, 70, 512, 512, True, True, (-1, -1)),
    (1, 2, 2, 64, 257, 128, 128, False, False, (10, 20)),
    (1, 2, 1, 300, 300, 64, 64, True, False, (50, -1)),     # tiles whose first and last key blocks are all masked
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[3]}x{c[4]}d{c[5]}{'c' if c[7] else 'n'}"
                         f"{'s' if c[8] else ''}w{c[9][0]}_{c[9][1]}")
def test_extras(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    announce(f"extras {case}")
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=Tq + 5 * Tk + dqk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    scale = 1 / math.sqrt(dqk)
    out, lse = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, window=window)
    p = torch.full((B, H, Tq, Tk), float("nan"), device="cuda")
    rm = torch.full((B, H, Tq), float("nan"), device="cuda")
    A.dense_extras(q, k, v, out, lse, causal=causal, scale=scale, sinks=sk, window=window, p=p, row_max=rm)
    torch.cuda.synchronize()
    rp, rrm = oracle.dense_attention_extras(inp["q"], inp["k"], scale=scale, causal=causal, sinks=inp["sinks"],
                                            window=window)
    ep = float(np.nan_to_num(np.abs(_np(p) - rp), nan=np.inf).max())
    em = _lse_err(_np(rm), rrm)
    assert ep <= TOL_P and em <= TOL_MAX, f"max|dp|={ep:.3e} max|drow_max|={em:.3e}"


def test_extras_one_output_and_strided():
    """Only row_max, then only p into a padded buffer: the same values."""
    announce("extras single outputs")
    inp = synth.randn_dense(1, 4, 2, 100, 100, 128, 128, dtype="bf16", sinks=True, seed=9)
    q, k, v, sk = (inp[n].cuda() for n in ("q", "k", "v", "sinks"))
    out, lse = A.dense(q, k, v, causal=True, scale=0.1, sinks=sk)
    p_full, rm_full = A.dense_extras(q, k, v, out, lse, causal=True, scale=0.1, sinks=sk)
    _, rm = A.dense_extras(q, k, v, out, lse, causal=True, scale=0.1, sinks=sk, want_p=False)
    big = torch.zeros((1, 4, 100, 128), device="cuda")
    p, _ = A.dense_extras(q, k, v, out, lse, causal=True, scale=0.1, sinks=sk, want_row_max=False,
                          p=big[..., :100])
    torch.cuda.synchronize()
    assert torch.equal(rm, rm_full) and torch.equal(p, p_full)
    assert float(big[..., 100:].abs().max()) == 0.0       # nothing written past Tk


def test_extras_rejects():
    q = torch.zeros(1, 2, 8, 96, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 8, device="cuda")
    with pytest.raises((A.AttnUnsupported, A.AttnInvalidArgument)):
        A.dense_extras(q, q, q, q, lse, causal=True, scale=0.1)
    torch.cuda.synchronize()
