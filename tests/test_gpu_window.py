"""Sliding-window forward (window_left, window_right) against the fp64 oracle.

Same tolerances as every dense case: max |O - O_ref| <= 2e-2, max |lse - lse_ref| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_parity import TOL_LSE, TOL_O, _lse_err, _np, _o_err, announce

pytestmark = pytest.mark.gpu


def run(inp, *, causal, scale, window, split=None):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    B, H, Tq, _ = q.shape
    out = torch.full((B, H, Tq, v.shape[-1]), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    if split is None:
        A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, out=out, lse=lse, window=window)
    else:
        A.dense_splitkv(q, k, v, causal=causal, scale=scale, sinks=sk, out=out, lse=lse, window=window,
                        n_splits=split)
    torch.cuda.synchronize()
    return out, lse


def check(inp, *, causal, scale, window, label, split=None):
    announce(f"window {label} q{tuple(inp['q'].shape)} k{tuple(inp['k'].shape)} causal={causal} "
             f"window={window} split={split}")
    out, lse = run(inp, causal=causal, scale=scale, window=window, split=split)
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=scale, causal=causal,
                                    sinks=inp["sinks"], window=window)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{label}: max|dO|={eo:.3e} max|dlse|={el:.3e}"


HEAD_DIMS = [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)]
WINDOWS = [(0, -1), (37, -1), (100, 0), (5, 70), (-1, 33)]


@pytest.mark.parametrize("dqk,dv", HEAD_DIMS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", WINDOWS, ids=lambda w: f"w{w[0]}_{w[1]}")
def test_window_head_dims(dqk, dv, causal, window):
    inp = synth.randn_dense(1, 4, 2, 300, 300, dqk, dv, dtype="bf16", sinks=dqk == 512, seed=dqk + 3 * window[0])
    check(inp, causal=causal, scale=1 / math.sqrt(dqk), window=window, label=f"d{dqk}/{dv}")


CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks, window
    (2, 8, 2, 100, 700, 128, 128, True, True, (150, -1)),     # Tq < Tk, rows near the end
    (1, 4, 4, 200, 90, 128, 128, True, False, (20, -1)),      # Tq > Tk: rows that see no key
    (1, 64, 1, 37, 37, 128, 128, True, True, (8, -1)),        # folded tiles straddling heads
    (1, 8, 8, 513, 513, 192, 128, False, False, (64, 64)),    # symmetric local window
    (1, 4, 1, 129, 129, 64, 64, True, False, (2000, -1)),     # wider than the keys: causal
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[3]}x{c[4]}d{c[5]}w{c[9][0]}_{c[9][1]}")
def test_window_cases(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=Tq + Tk)
    check(inp, causal=causal, scale=1 / math.sqrt(dqk), window=window, label=str(case))


@pytest.mark.parametrize("n", [0, 3, 9])
def test_window_splitkv(n):
    """Decode with a window over a long cache, through the split-KV path."""
    inp = synth.randn_dense(2, 16, 2, 1, 5000, 128, 128, dtype="bf16", sinks=True, seed=77 + n)
    check(inp, causal=True, scale=1 / math.sqrt(128), window=(1500, -1), label="decode", split=n)


def test_window_large_causal_equals_causal():
    """A window wider than every row's causal reach gives exactly the causal result."""
    announce("window wide == causal")
    inp = synth.randn_dense(1, 8, 2, 333, 333, 128, 128, dtype="bf16", sinks=False, seed=5)
    a = run(inp, causal=True, scale=0.1, window=(-1, -1))
    b = run(inp, causal=True, scale=0.1, window=(400, 7))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_window_rejects():
    inp = synth.randn_dense(1, 4, 2, 16, 16, 64, 64, dtype="f32", sinks=False, seed=1)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    with pytest.raises(A.AttnUnsupported):
        A.dense(q, k, v, causal=True, scale=0.1, window=(4, -1))
    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    with pytest.raises(A.AttnInvalidArgument):
        A.dense(qb, kb, vb, causal=True, scale=0.1, window=(-2, -1))
    torch.cuda.synchronize()


def test_window_full_workload_sampled():
    """The benchmark's sliding-window launch at full size, sampled rows against the oracle."""
    s = synth.spec(7)
    announce(f"window full workload {s.name}")
    inp = synth.make(7)
    out, lse = run(inp, causal=s.causal, scale=s.scale, window=s.window)
    rng = np.random.default_rng(7)
    rows = [(int(rng.integers(s.B)), int(rng.integers(s.H)), int(t))
            for t in list(rng.integers(0, s.Tq, 48)) + [0, s.window[0], s.Tq - 1]]
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=s.scale, causal=s.causal,
                                    sinks=inp["sinks"], rows=rows, window=s.window)
    go = np.stack([_np(out[b, h, t]) for b, h, t in rows])
    gl = np.array([float(lse[b, h, t]) for b, h, t in rows])
    eo, el = _o_err(go, ro), _lse_err(gl, rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"
