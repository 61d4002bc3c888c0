"""Decode over a quantized K/V cache (attn_fwd_dense_qkv) against the fp64 oracle.

The oracle decodes the same cache bytes from the block format and runs the
definition. The kernel decodes to f16 (11 significant bits; a q8_0 value d*q
needs up to 18), so its K/V differ from the exact decode by at most 2^-11
relative: same tolerances as the dense path, max |O - O_ref| <= 2e-2,
max |lse - lse_ref| <= 1e-3.
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


def run(inp, *, causal, scale, n_splits=0):
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    B, H, Tq, d = q.shape
    out = torch.full((B, H, Tq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    A.dense_qkv(q, k, v, fmt=inp["fmt"], causal=causal, scale=scale, sinks=sk, n_splits=n_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def reference(inp, *, causal, scale):
    kd = oracle.dequantize_rows(inp["k"], inp["fmt"])
    vd = oracle.dequantize_rows(inp["v"], inp["fmt"])
    return oracle.dense_attention(inp["q"], kd, vd, scale=scale, causal=causal, sinks=inp["sinks"])


CASES = [
    # B, H, Hkv, Tq, Tk, causal, sinks, n_splits
    (4, 32, 8, 4, 2000, True, False, 0),      # multi-sequence decode, 4 tokens per sequence
    (2, 8, 2, 1, 777, True, True, 0),         # single-token decode, ragged cache
    (1, 8, 1, 16, 300, True, True, 5),        # 128 folded rows, uneven ranges
    (1, 4, 4, 7, 65, False, False, 1),        # one range: direct output
    (1, 2, 1, 40, 30, True, False, 0),        # Tq > Tk: rows that see no key
    (3, 4, 2, 3, 33, True, True, 100),        # more ranges asked than key blocks
    (1, 8, 2, 1, 6000, True, True, 70),       # many ranges: several merge batches
    (2, 64, 1, 1, 700, True, True, 0),        # MQA decode: 64 rows of one kv head, one workgroup's tiles
    (1, 32, 1, 1, 500, True, False, 3),       # 32 rows: two row tiles
    (1, 8, 1, 5, 300, True, False, 0),        # 40 rows: a partly filled row tile, one empty
]


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}x{c[4]}"
                         f"{'c' if c[5] else 'n'}{'s' if c[6] else ''}n{c[7]}")
def test_qkv_matches_oracle(case, fmt, d):
    B, H, Hkv, Tq, Tk, causal, sinks, n = case
    announce(f"qkv {fmt} d{d} {case}")
    inp = synth.make_quant_kv(B, H, Hkv, Tq, Tk, d, fmt, seed=Tq * 13 + Tk + d, sinks=sinks)
    scale = 1 / math.sqrt(d)
    out, lse = run(inp, causal=causal, scale=scale, n_splits=n)
    ro, rl = reference(inp, causal=causal, scale=scale)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{fmt} {case}: max|dO|={eo:.3e} max|dlse|={el:.3e}"


def test_qkv_dispatch_no_conversion():
    """The quantized path runs its own kernel (and the merge); no other kernel path
    (such as a bf16 forward over a converted cache) runs."""
    inp = synth.make_quant_kv(2, 8, 2, 2, 600, 128, "q8_0", seed=1)
    A.reset_dispatch_counts()
    run(inp, causal=True, scale=0.1, n_splits=4)
    assert A.dispatch_count("dense_qkv_q8_0_d128") == 1
    assert A.dispatch_count("splitkv_merge") == 1
    for path in ("dense_bf16_d128", "dense_qkv_q4_0_d128"):
        assert A.dispatch_count(path) == 0


@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_qkv_dispatch_wide(fmt, d):
    """256- and 512-wide heads run their own kernel paths (and no other width's)."""
    inp = synth.make_quant_kv(1, 8, 2, 2, 300, d, fmt, seed=3)
    A.reset_dispatch_counts()
    out, lse = run(inp, causal=True, scale=1 / math.sqrt(d), n_splits=2)
    for other in (128, 256, 512):
        assert A.dispatch_count(f"dense_qkv_{fmt}_d{other}") == (1 if other == d else 0)
    ro, rl = reference(inp, causal=True, scale=1 / math.sqrt(d))
    assert _o_err(_np(out), ro) <= TOL_O and _lse_err(_np(lse), rl) <= TOL_LSE


def test_qkv_rejects():
    inp = synth.make_quant_kv(1, 4, 2, 2, 64, 128, "q8_0", seed=2)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    with pytest.raises(A.AttnUnsupported):
        A.dense_qkv(q, k, v, fmt="q5_0", causal=True)
    with pytest.raises(A.AttnInvalidArgument):   # row bytes do not match the format
        A.dense_qkv(q, k[..., :68], v[..., :68], fmt="q8_0", causal=True)
    odd = synth.make_quant_kv(1, 4, 2, 2, 64, 384, "q8_0", seed=4)
    with pytest.raises(A.AttnUnsupported):       # 384-wide heads are not compiled
        A.dense_qkv(odd["q"].cuda(), odd["k"].cuda(), odd["v"].cuda(), fmt="q8_0", causal=True)
    torch.cuda.synchronize()


def test_qkv_full_workload_sampled():
    """The benchmark's quantized decode launch at full size; sampled rows against the oracle."""
    s = synth.QUANT_DECODE
    announce(f"qkv full workload {s}")
    inp = synth.make_quant_kv(s["B"], s["H"], s["Hkv"], s["Tq"], s["Tk"], s["d"], s["fmt"], seed=s["seed"])
    scale = 1 / math.sqrt(s["d"])
    out, lse = run(inp, causal=True, scale=scale)
    kd = oracle.dequantize_rows(inp["k"], inp["fmt"])
    vd = oracle.dequantize_rows(inp["v"], inp["fmt"])
    rng = np.random.default_rng(8)
    rows = [(int(rng.integers(s["B"])), int(rng.integers(s["H"])), int(rng.integers(s["Tq"]))) for _ in range(24)]
    ro, rl = oracle.dense_attention(inp["q"], kd, vd, scale=scale, causal=True, rows=rows)
    go = np.stack([_np(out[b, h, t]) for b, h, t in rows])
    gl = np.array([float(lse[b, h, t]) for b, h, t in rows])
    eo, el = _o_err(go, ro), _lse_err(gl, rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("layout", ["padded_rows", "token_major"])
def test_qkv_strided_cache(fmt, layout):
    """Caches that are not [B, Hkv, Tk, row] back to back: rows padded by 12
    bytes, and the token-major [B, Tk, Hkv, row] layout viewed as [B, Hkv, Tk, row]."""
    B, H, Hkv, Tq, Tk, d = 2, 8, 2, 3, 333, 128
    announce(f"qkv strided {fmt} {layout}")
    inp = synth.make_quant_kv(B, H, Hkv, Tq, Tk, d, fmt, seed=17, sinks=True)
    rb = inp["k"].shape[-1]

    def restride(x):
        if layout == "padded_rows":
            buf = torch.zeros((B, Hkv, Tk, rb + 12), dtype=torch.uint8)
            buf[..., :rb] = x
            return buf.cuda()[..., :rb]
        return x.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)

    k, v = restride(inp["k"]), restride(inp["v"])
    assert not k.is_contiguous()
    out = torch.full((B, H, Tq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    A.dense_qkv(inp["q"].cuda(), k, v, fmt=fmt, causal=True, sinks=inp["sinks"].cuda(), out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = reference(inp, causal=True, scale=1 / math.sqrt(d))
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{fmt} {layout}: max|dO|={eo:.3e} max|dlse|={el:.3e}"
