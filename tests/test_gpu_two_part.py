"""MLA two-part rows (q/k no-rope part + rope part read in place) against the
fp64 oracle, and against the concatenated call of the same library.

Tolerances as the dense path (max |O - O_ref| <= 2e-2, max |lse - lse_ref| <= 1e-3).
The two-part kernel accumulates the same products in the same order as the
kernel on concatenated rows, so the two give identical bits.
"""
import math

import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_parity import TOL_LSE, TOL_O, _lse_err, _np, _o_err, announce

pytestmark = pytest.mark.gpu

DN, DR, DV = 128, 64, 128


def parts(B, H, Hkv, Tq, Tk, seed, shared, sinks=False):
    """Seeded dense inputs of width 192, cut into the two parts (strided views)."""
    s = synth.randn_dense(B, H, Hkv, Tq, Tk, DN + DR, DV, dtype="bf16", sinks=sinks, seed=seed)
    q, k, v = s["q"].cuda(), s["k"].cuda(), s["v"].cuda()
    qn, qr, kn = q[..., :DN], q[..., DN:], k[..., :DN]
    kr = k[:, :1, :, DN:].expand(B, Hkv, Tk, DR) if shared else k[..., DN:]
    sk = s["sinks"].cuda() if s["sinks"] is not None else None
    return qn, qr, kn, kr, v, sk


def check(B, H, Hkv, Tq, Tk, *, causal, shared, sinks=False, window=(-1, -1), seed=0):
    announce(f"two-part B={B} H={H}/{Hkv} Tq={Tq} Tk={Tk} causal={causal} shared={shared} sinks={sinks} "
             f"window={window}")
    qn, qr, kn, kr, v, sk = parts(B, H, Hkv, Tq, Tk, seed, shared, sinks)
    scale = 1 / math.sqrt(DN + DR)
    out, lse = A.dense(qn, kn, v, causal=causal, scale=scale, sinks=sk, window=window, q_rope=qr, k_rope=kr)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention_two_part(qn.cpu(), qr.cpu(), kn.cpu(), kr[:, :1].cpu() if shared else kr.cpu(),
                                             v.cpu(), scale=scale, causal=causal,
                                             sinks=None if sk is None else sk.cpu(), window=window)
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"
    # the concatenated rows through the one-pointer kernel: identical bits
    qc = torch.cat([qn, qr], dim=-1)
    kc = torch.cat([kn, kr], dim=-1)
    oc, lc = A.dense(qc, kc, v, causal=causal, scale=scale, sinks=sk, window=window)
    torch.cuda.synchronize()
    assert torch.equal(out, oc) and torch.equal(lse, lc)


CASES = [
    # B, H, Hkv, Tq, Tk, causal, shared, sinks, window
    (2, 4, 2, 200, 200, True, False, False, (-1, -1)),
    (1, 16, 16, 300, 300, False, True, False, (-1, -1)),
    (1, 8, 1, 130, 130, True, False, True, (-1, -1)),
    (1, 4, 4, 33, 301, True, True, True, (-1, -1)),      # Tq < Tk
    (1, 4, 2, 150, 40, True, False, False, (-1, -1)),    # Tq > Tk: rows that see no key
    (2, 4, 4, 257, 257, True, True, False, (64, -1)),    # sliding window
    (1, 2, 1, 1, 1, True, False, False, (-1, -1)),       # one query, one key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}x{c[4]}"
                         f"{'c' if c[5] else 'n'}{'sh' if c[6] else ''}{'s' if c[7] else ''}w{c[8][0]}")
def test_two_part_cases(case):
    B, H, Hkv, Tq, Tk, causal, shared, sinks, window = case
    check(B, H, Hkv, Tq, Tk, causal=causal, shared=shared, sinks=sinks, window=window, seed=Tq + 7 * Tk)


def test_two_part_splitkv_decode():
    """The split-KV path with two-part rows: one query row per head over a long cache."""
    announce("two-part split-KV decode")
    qn, qr, kn, kr, v, sk = parts(2, 16, 1, 1, 3000, 77, True, True)
    scale = 1 / math.sqrt(DN + DR)
    out, lse = A.dense_splitkv(qn, kn, v, causal=True, scale=scale, sinks=sk, q_rope=qr, k_rope=kr, n_splits=8)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention_two_part(qn.cpu(), qr.cpu(), kn.cpu(), kr[:, :1].cpu(), v.cpu(), scale=scale,
                                             causal=True, sinks=sk.cpu())
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"


def test_two_part_full_workload():
    """The MLA workload (B4 H16 T4096, causal) with the rope key shared by the heads:
    sampled rows against the oracle, all rows against the concatenated call."""
    s = synth.spec(3)
    announce(f"two-part full workload {s.name}")
    inp = synth.make(3)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    qn, qr, kn = q[..., :DN], q[..., DN:], k[..., :DN]
    kr = k[:, :1, :, DN:].expand(s.B, s.Hkv, s.Tk, DR)
    out, lse = A.dense(qn, kn, v, causal=True, scale=s.scale, q_rope=qr, k_rope=kr)
    oc, lc = A.dense(torch.cat([qn, qr], -1), torch.cat([kn, kr], -1), v, causal=True, scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, oc) and torch.equal(lse, lc)
    rows = [(0, 0, 0), (1, 5, 1), (2, 9, 777), (3, 15, 4095), (3, 3, 2048)]
    kc = torch.cat([k[..., :DN], k[:, :1, :, DN:].expand(s.B, s.Hkv, s.Tk, DR)], -1).cpu()
    ro, rl = oracle.dense_attention(q.cpu(), kc, v.cpu(), scale=s.scale, causal=True, rows=rows)
    got_o = torch.stack([out[b, h, t] for b, h, t in rows])
    got_l = torch.stack([lse[b, h, t] for b, h, t in rows])
    eo, el = _o_err(_np(got_o), ro), _lse_err(_np(got_l), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"max|dO|={eo:.3e} max|dlse|={el:.3e}"


def test_two_part_rejects():
    qn = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnUnsupported):        # d_qk = 64 + 32 has no two-part kernel
        A.dense(qn[..., :64], kn[..., :64], kn, q_rope=qr[..., :32], k_rope=kr[..., :32])
    with pytest.raises(A.AttnInvalidArgument):    # q_rope without k_rope
        A.dense(qn, kn, kn, q_rope=qr)
    torch.cuda.synchronize()
