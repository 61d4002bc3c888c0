"""Sparse top-k decode over an fp8 pool (attn_fwd_sparse_fp8) against the fp64
oracle on the decoded pool.

The kernel multiplies exactly decoded E4M3 codes (4 significant bits, exact in
bf16) and applies each key's per-block scale in fp32, so the inputs of its
products carry no rounding beyond the bf16 q and P of the dense paths: the same
bars, max |O - O_ref| <= 2e-2 and max |lse - lse_ref| <= 1e-3.
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


def run_and_check(inp, idx, *, n_splits=0, label=""):
    q, codes, scales = inp["q"], inp["codes"], inp["scales"]
    sk = inp["sinks"]
    scale = 1 / math.sqrt(512)
    out = torch.full((q.shape[0], 64, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((q.shape[0], 64), float("nan"), device="cuda")
    A.sparse_fp8(q.cuda(), codes.cuda(), scales.cuda(), idx.cuda(), scale=scale,
                 sinks=None if sk is None else sk.cuda(), n_splits=n_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    pool = oracle.dequantize_fp8_rows(codes.numpy(), scales.numpy())
    ro, rl = oracle.sparse_topk_attention(q, pool, idx.numpy(), d_v=512, scale=scale, sinks=sk)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{label}: max|dO|={eo:.3e} max|dlse|={el:.3e}"
    return out, lse


CASES = [
    # Sq, N, topk, sinks, n_splits, special
    (1, 300, 64, False, 0, False),
    (5, 300, 100, True, 0, True),      # a ragged last step, duplicates, skipped slots
    (3, 5000, 2048, True, 0, False),   # several ranges chosen by the library
    (2, 5000, 2048, False, 3, False),  # uneven ranges
    (33, 1000, 257, True, 1, True),    # one range
    (4, 70000, 4096, False, 1, False), # the largest range (the kernel's index buffer)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Sq{c[0]}N{c[1]}k{c[2]}{'s' if c[3] else ''}n{c[4]}"
                         f"{'x' if c[5] else ''}")
def test_sparse_fp8_cases(case):
    Sq, N, topk, sinks, n_splits, special = case
    announce(f"sparse fp8 {case}")
    inp = synth.make_sparse_fp8(Sq, 64, N, 512, topk, seed=Sq + topk, sinks=sinks)
    idx = inp["idx"].clone()
    if special:
        idx[:, 1] = idx[:, 0]
        idx[0, 2] = -1
        idx[min(1, Sq - 1), 3] = N + 7
    run_and_check(inp, idx, n_splits=n_splits, label=str(case))


def test_sparse_fp8_no_slot():
    """Every slot skipped: out = 0, lse = the sink (or -inf)."""
    announce("sparse fp8 all skipped")
    inp = synth.make_sparse_fp8(2, 64, 100, 512, 40, seed=5, sinks=True)
    idx = torch.full((2, 40), -1, dtype=torch.int32)
    out, lse = run_and_check(inp, idx)
    assert float(out.float().abs().max()) == 0.0
    assert torch.equal(lse.cpu(), inp["sinks"][None, :].expand(2, 64))


def test_sparse_fp8_full_decode_sampled():
    """The benchmark's decode step (128 queries x 64 heads, top-k 2048 of 65536 rows):
    sampled queries against the oracle."""
    s = synth.SPARSE_FP8_DECODE
    announce(f"sparse fp8 full decode {s}")
    inp = synth.make_sparse_fp8(s["Sq"], s["Hq"], s["N"], s["d"], s["topk"], seed=s["seed"])
    scale = 1 / math.sqrt(s["d"])
    out, lse = A.sparse_fp8(inp["q"].cuda(), inp["codes"].cuda(), inp["scales"].cuda(), inp["idx"].cuda(),
                            scale=scale)
    torch.cuda.synchronize()
    pool = oracle.dequantize_fp8_rows(inp["codes"].numpy(), inp["scales"].numpy())
    qs = [0, 77, s["Sq"] - 1]
    ro, rl = oracle.sparse_topk_attention(inp["q"], pool, inp["idx"].numpy(), d_v=512, scale=scale, queries=qs)
    eo, el = _o_err(_np(out[qs]), ro), _lse_err(_np(lse[qs]), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"
    assert A.dispatch_count("sparse_fp8_d512") > 0


def test_sparse_fp8_rejects():
    q = torch.zeros(2, 32, 512, dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros(10, 512, dtype=torch.uint8, device="cuda")
    scales = torch.ones(10, 4, device="cuda")
    idx = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(A.AttnUnsupported):       # 64 heads only
        A.sparse_fp8(q, codes, scales, idx)
    torch.cuda.synchronize()
