"""Packed variable-length forward (attn_fwd_varlen) against the fp64 oracle.

Same tolerances as the dense path: max |O - O_ref| <= 2e-2, max |lse - lse_ref| <= 1e-3
(rows of empty sequences are never written; lse rows the oracle leaves at -inf are
compared only where a sequence owns them).
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


def packed(lq, lk, H, Hkv, dqk, dv, seed, sinks=False):
    """Seeded packed inputs: the dense recipe for one long sequence of each side, cut."""
    s = synth.randn_dense(1, H, Hkv, max(1, sum(lq)), max(1, sum(lk)), dqk, dv, dtype="bf16", sinks=sinks, seed=seed)
    q = s["q"][0, :, :sum(lq)].transpose(0, 1).contiguous()      # [total_q, H, d]
    k = s["k"][0, :, :sum(lk)].transpose(0, 1).contiguous()
    v = s["v"][0, :, :sum(lk)].transpose(0, 1).contiguous()
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    return q, k, v, cq, ck, s["sinks"]


def check(lq, lk, H, Hkv, dqk, dv, *, causal, window=(-1, -1), sinks=False, seed=0):
    announce(f"varlen lq={lq} lk={lk} H={H}/{Hkv} d={dqk}/{dv} causal={causal} window={window} sinks={sinks}")
    q, k, v, cq, ck, sk = packed(lq, lk, H, Hkv, dqk, dv, seed, sinks)
    scale = 1 / math.sqrt(dqk)
    out = torch.full((q.shape[0], H, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    A.dense_varlen(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(),
                   max(lq), causal=causal, scale=scale, sinks=None if sk is None else sk.cuda(), window=window,
                   out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention_varlen(q, k, v, cq, ck, scale=scale, causal=causal, sinks=sk, window=window)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"


@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_head_dims(dqk, dv, causal):
    lq = [130, 7, 300, 64]
    check(lq, lq, 4, 2, dqk, dv, causal=causal, sinks=dqk == 256, seed=dqk)


CASES = [
    # lq, lk, H, Hkv, causal, window, sinks
    ([1, 1, 1, 1], [900, 33, 1, 257], 8, 2, True, (-1, -1), True),        # decode-like rows, ragged caches
    ([100, 0, 37, 256], [300, 5, 37, 256], 8, 8, True, (-1, -1), False),  # an empty sequence, Tq < Tk
    ([200, 50], [40, 50], 4, 1, True, (-1, -1), False),                  # Tq > Tk: rows that see no key
    ([513, 1, 255], [513, 1, 255], 16, 4, True, (64, -1), True),         # sliding window per sequence
    ([77, 300], [77, 300], 4, 2, False, (20, 20), False),                # local window, non-causal
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"lq{sum(c[0])}lk{sum(c[1])}H{c[2]}/{c[3]}"
                         f"{'c' if c[4] else 'n'}w{c[5][0]}_{c[5][1]}")
def test_varlen_cases(case):
    lq, lk, H, Hkv, causal, window, sinks = case
    check(lq, lk, H, Hkv, 128, 128, causal=causal, window=window, sinks=sinks, seed=sum(lq) + 7 * sum(lk))


def test_varlen_equals_padded_batch():
    """Equal lengths: the packed call gives the dense batched call's bits."""
    announce("varlen == padded batch")
    s = synth.randn_dense(3, 8, 2, 200, 200, 128, 128, dtype="bf16", sinks=True, seed=4)
    q, k, v, sk = (s[n].cuda() for n in ("q", "k", "v", "sinks"))
    out, lse = A.dense(q, k, v, causal=True, scale=0.1, sinks=sk)
    pq = q.transpose(1, 2).reshape(600, 8, 128).contiguous()
    pk = k.transpose(1, 2).reshape(600, 2, 128).contiguous()
    pv = v.transpose(1, 2).reshape(600, 2, 128).contiguous()
    cu = torch.tensor([0, 200, 400, 600], dtype=torch.int32, device="cuda")
    o2, l2 = A.dense_varlen(pq, pk, pv, cu, cu, 200, causal=True, scale=0.1, sinks=sk)
    torch.cuda.synchronize()
    assert torch.equal(o2, out.transpose(1, 2).reshape(600, 8, 128))
    assert torch.equal(l2, lse.permute(1, 0, 2).reshape(8, 600))


def test_varlen_rejects():
    q = torch.zeros(10, 4, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(10, 2, 128, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    with pytest.raises(A.AttnUnsupported):
        A.dense_varlen(q.float(), k.float(), k.float(), cu, cu, 10)
    q5 = torch.zeros(10, 4, 512, dtype=torch.bfloat16, device="cuda")
    k5 = torch.zeros(10, 1, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnUnsupported):       # the 512-wide kernel has no packed mode
        A.dense_varlen(q5, k5, k5, cu, cu, 10)
    with pytest.raises(A.AttnInvalidArgument):
        A.dense_varlen(q, k, k, cu.long(), cu, 10)
    with pytest.raises(A.AttnInvalidArgument):
        A.dense_varlen(q, k, k, cu, torch.tensor([0, 5, 10], dtype=torch.int32, device="cuda"), 10)
    torch.cuda.synchronize()


def test_varlen_full_workload_sampled():
    """The benchmark's packed batch at full size. The oracle checks the shortest sequence
    (every row of kv head 3's query heads) and sampled rows of the longest one (a causal
    row t of a sequence is the last row of attention over that sequence's keys [0, t])."""
    s = synth.VARLEN_PREFILL
    announce(f"varlen full workload {s}")
    inp = synth.make_varlen(s)
    lens, cu = inp["lens"], inp["cu"]
    H, Hkv, d = s["H"], s["Hkv"], s["d"]
    g = H // Hkv
    scale = 1 / math.sqrt(d)
    out, lse = A.dense_varlen(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), torch.from_numpy(cu).cuda(),
                              torch.from_numpy(cu).cuda(), int(lens.max()), causal=True, scale=scale)
    torch.cuda.synchronize()
    out, lse = _np(out), _np(lse)

    def seq(x, i):
        return x[cu[i]:cu[i + 1]].transpose(0, 1)[None]      # [1, heads, L, d]

    i = int(np.argmin(lens))
    kvh = 3
    hs = slice(kvh * g, (kvh + 1) * g)
    ro, rl = oracle.dense_attention(seq(inp["q"], i)[:, hs], seq(inp["k"], i)[:, kvh:kvh + 1],
                                    seq(inp["v"], i)[:, kvh:kvh + 1], scale=scale, causal=True)
    eo = _o_err(out[cu[i]:cu[i + 1], hs].transpose(1, 0, 2)[None], ro)
    el = _lse_err(lse[hs, cu[i]:cu[i + 1]][None], rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"shortest sequence: max|dO|={eo:.3e} max|dlse|={el:.3e}"
    j = int(np.argmax(lens))
    qj, kj, vj = seq(inp["q"], j), seq(inp["k"], j), seq(inp["v"], j)
    for t in (0, 1, 777, int(lens[j]) // 2, int(lens[j]) - 1):
        ro, rl = oracle.dense_attention(qj[:, :, t:t + 1], kj[:, :, :t + 1], vj[:, :, :t + 1], scale=scale,
                                        causal=True)
        eo = _o_err(out[cu[j] + t][None, :, None, :], ro)
        el = _lse_err(lse[:, cu[j] + t][None, :, None], rl)
        assert eo <= TOL_O and el <= TOL_LSE, f"longest sequence row {t}: max|dO|={eo:.3e} max|dlse|={el:.3e}"
