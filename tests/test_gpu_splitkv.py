"""Split-KV dense forward (attn_fwd_dense_splitkv) against the fp64 oracle.

The split path must give the same attention as the definition: the key
ranges and the merge are an evaluation order, not a different result.
Tolerances as for the dense path: max |O - O_ref| <= 2e-2, max |lse - lse_ref| <= 1e-3.
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


def run_split(inp, *, causal, scale, n_splits):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    B, H, Tq, _ = q.shape
    out = torch.full((B, H, Tq, v.shape[-1]), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    A.dense_splitkv(q, k, v, causal=causal, scale=scale, sinks=sk, n_splits=n_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks, n_splits
    (2, 8, 2, 1, 1000, 128, 128, True, True, 0),      # GQA decode, library's choice
    (2, 8, 2, 1, 1000, 128, 128, True, False, 3),     # uneven ranges
    (2, 8, 2, 1, 1000, 128, 128, False, False, 100),  # more ranges asked than key blocks
    (1, 64, 1, 1, 3000, 512, 512, True, True, 0),     # MQA d512 decode with sinks
    (1, 4, 1, 37, 1300, 192, 128, True, False, 0),    # short prefill: early rows see few ranges
    (1, 4, 1, 37, 1300, 192, 128, True, True, 5),
    (2, 4, 4, 5, 777, 64, 64, False, True, 7),        # non-causal, ragged last range
    (1, 8, 2, 40, 30, 128, 128, True, True, 2),       # Tq > Tk: rows that see no key
    (1, 8, 2, 3, 900, 256, 256, True, False, 4),      # d256 (one-group kernel)
    (1, 4, 1, 1, 20000, 64, 64, True, True, 150),     # many ranges: several merge batches per lane
    (1, 8, 1, 2, 12000, 512, 512, True, False, 40),   # wide rows: two merge passes, three batches
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}x{c[4]}d{c[5]}/{c[6]}"
                         f"{'c' if c[7] else 'n'}{'s' if c[8] else ''}n{c[9]}")
def test_splitkv_matches_oracle(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, n = case
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=Tq * 7919 + Tk + dqk)
    scale = 1 / math.sqrt(dqk)
    announce(f"split-KV {case}")
    A.reset_dispatch_counts()
    out, lse = run_split(inp, causal=causal, scale=scale, n_splits=n)
    chosen = n if n else A.splitkv_choose(B, H, Hkv, Tq, Tk, dqk, dv, causal=causal, sinks=sinks)
    if A.splitkv_workspace_bytes(B, H, Hkv, Tq, Tk, dqk, dv, n_splits=n, causal=causal, sinks=sinks) > 0:
        assert A.dispatch_count("splitkv_merge") == 1, "the split path (and its merge) must have run"
    else:
        assert A.dispatch_count("splitkv_merge") == 0
    assert chosen >= 1
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=scale, causal=causal, sinks=inp["sinks"])
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"split-KV: max|dO|={eo:.3e} max|dlse|={el:.3e}"


def test_splitkv_one_range_is_the_plain_path():
    """A single range launches exactly the plain kernel and no merge."""
    inp = synth.randn_dense(1, 8, 2, 64, 100, 128, 128, dtype="bf16", seed=3)
    A.reset_dispatch_counts()
    o1, l1 = run_split(inp, causal=True, scale=0.1, n_splits=1)
    assert A.dispatch_count("dense_bf16_d128") == 1 and A.dispatch_count("splitkv_merge") == 0
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o2, l2 = A.dense(q, k, v, causal=True, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_deterministic_and_workspace_reuse():
    """Two calls on one workspace, the second with a smaller problem, repeat bitwise."""
    big = synth.randn_dense(1, 64, 1, 1, 4000, 512, 512, dtype="bf16", sinks=True, seed=11)
    small = synth.randn_dense(1, 8, 1, 2, 700, 512, 512, dtype="bf16", sinks=True, seed=12)
    ws = torch.empty(A.splitkv_workspace_bytes(1, 64, 1, 1, 4000, 512, 512, sinks=True), dtype=torch.uint8,
                     device="cuda")
    res = []
    for inp in (big, small, big):
        q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
        o, l = A.dense_splitkv(q, k, v, causal=True, sinks=inp["sinks"].cuda(), workspace=ws)
        torch.cuda.synchronize()
        res.append((o.clone(), l.clone()))
    assert torch.equal(res[0][0], res[2][0]) and torch.equal(res[0][1], res[2][1])
    ro, rl = oracle.dense_attention(small["q"], small["k"], small["v"], scale=1 / math.sqrt(512), causal=True,
                                    sinks=small["sinks"])
    assert _o_err(_np(res[1][0]), ro) <= TOL_O and _lse_err(_np(res[1][1]), rl) <= TOL_LSE
