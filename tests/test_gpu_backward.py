"""Dense backward (attn_bwd_dense) against the fp64 oracle's gradients.

The GPU forward supplies out and lse (as in training); the oracle computes the
exact gradients of the same bf16 inputs from the definition. Tolerance, from
the arithmetic: P and dS enter the MFMAs as bf16 (relative rounding 2^-9 each)
and every gradient is rounded once to bf16, so the error of a gradient tensor
is a few 2^-9 of its largest entry; the bar is max |g - g_ref| <= 2e-2 * max|g_ref|
(about 10x that), and 1e-2 relative for the fp32 sink gradients (computed from
the bf16 output through D). Gradients that vanish exactly (one key: P = 1 and
dS = dP - D = 0) keep the rounding of O in D, a few 2^-9 of |dO.v| ~ 1: the
scale of the bar never drops below 0.05 (an absolute floor of 1e-3).
"""
import math

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth
from test_gpu_parity import _np, announce

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2
TOL_SINK = 1e-2


def _rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 0.05)
    d = np.abs(np.asarray(got, np.float64) - ref)
    return float(np.nan_to_num(d, nan=np.inf).max()) / scale if d.size else 0.0


def run_fwd_bwd(inp, dout, *, causal, scale):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    out, lse = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk)
    d = dout.cuda()
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    res = A.dense_backward(q, k, v, out, d, lse, causal=causal, scale=scale, sinks=sk, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def check_bwd(inp, dout, *, causal, scale, label):
    announce(f"bwd {label} q{tuple(inp['q'].shape)} k{tuple(inp['k'].shape)} v{tuple(inp['v'].shape)} "
             f"causal={causal} sinks={inp['sinks'] is not None}")
    dq, dk, dv, ds = run_fwd_bwd(inp, dout, causal=causal, scale=scale)
    rq, rk, rv, rs = oracle.dense_attention_backward(inp["q"], inp["k"], inp["v"], dout, scale=scale, causal=causal,
                                                     sinks=inp["sinks"])
    errs = {"dq": _rel_err(_np(dq), rq), "dk": _rel_err(_np(dk), rk), "dv": _rel_err(_np(dv), rv)}
    assert max(errs.values()) <= TOL_REL, f"{label}: {errs}"
    if rs is not None:
        es = _rel_err(_np(ds), rs)
        assert es <= TOL_SINK, f"{label}: dsinks rel err {es:.3e}"
    return errs


BWD_DIMS = [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)]


@pytest.mark.parametrize("dqk,dv", BWD_DIMS)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_head_dims(dqk, dv, causal):
    # T = 200: several 64-row query steps and 128-key blocks, ragged in both
    inp = synth.randn_dense(2, 4, 2, 200, 200, dqk, dv, dtype="bf16", sinks=False, seed=dqk + dv + 7)
    dout = synth.randn_dout(2, 4, 200, dv, seed=dqk + dv + 7)
    check_bwd(inp, dout, causal=causal, scale=1 / math.sqrt(dqk), label=f"d{dqk}/{dv}")


CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks
    (1, 8, 1, 130, 130, 128, 128, True, True),     # MQA with sinks
    (1, 8, 2, 33, 300, 128, 128, True, False),     # Tq < Tk: bottom-right causal
    (1, 4, 4, 150, 40, 64, 64, True, True),        # Tq > Tk: rows that see no key
    (2, 6, 3, 1, 257, 192, 128, True, True),       # one query row
    (1, 2, 1, 97, 1, 128, 128, False, False),      # one key: dq = dk = 0
    (1, 16, 16, 64, 64, 192, 128, True, False),    # MLA shape, exact tiles
    (1, 8, 1, 130, 130, 512, 512, True, True),     # MQA, 512-wide heads, sinks
    (1, 8, 2, 70, 333, 256, 256, True, True),      # GQA, 256-wide heads, Tq < Tk, sinks
    (1, 4, 4, 150, 40, 512, 512, True, False),     # 512-wide, rows that see no key
    (2, 6, 3, 1, 257, 256, 256, False, True),      # 256-wide, one query row
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}x{c[4]}d{c[5]}/{c[6]}"
                         f"{'c' if c[7] else 'n'}{'s' if c[8] else ''}")
def test_bwd_cases(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks = case
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=Tq * 31 + Tk)
    dout = synth.randn_dout(B, H, Tq, dv, seed=Tq * 31 + Tk)
    check_bwd(inp, dout, causal=causal, scale=1 / math.sqrt(dqk), label=str(case))


def test_bwd_no_keys():
    """Tk = 0: out = 0, so dq = 0 and the sink gradient is 0."""
    announce("bwd Tk=0")
    inp = synth.randn_dense(1, 4, 2, 9, 0, 128, 128, dtype="bf16", sinks=True, seed=5)
    dout = synth.randn_dout(1, 4, 9, 128, seed=5)
    dq, dk, dv, ds = run_fwd_bwd(inp, dout, causal=True, scale=0.1)
    assert float(dq.float().abs().max()) == 0.0
    assert float(ds.abs().max()) == 0.0


@pytest.mark.parametrize("d", [256, 512])
def test_bwd_wide_empty(d):
    """256/512-wide heads at the edges: no keys (dq = 0, dsinks = 0), no queries
    (dk = dv = 0, with the heads split), one query row per head."""
    announce(f"bwd d{d} empty edges")
    inp = synth.randn_dense(1, 8, 1, 9, 0, d, d, dtype="bf16", sinks=True, seed=d + 1)
    dout = synth.randn_dout(1, 8, 9, d, seed=d + 1)
    dq, dk, dv, ds = run_fwd_bwd(inp, dout, causal=True, scale=0.05)
    assert float(dq.float().abs().max()) == 0.0 and float(ds.abs().max()) == 0.0
    q = torch.zeros(1, 8, 0, d, dtype=torch.bfloat16, device="cuda")
    k = synth.randn_dense(1, 8, 1, 1, 40, d, d, dtype="bf16", sinks=False, seed=3)["k"].cuda()
    out = torch.zeros_like(q)
    lse = torch.zeros(1, 8, 0, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    A.dense_backward(q, k, k, out, out, lse, causal=False, scale=0.05, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert float(dk.float().abs().max()) == 0.0 and float(dv.float().abs().max()) == 0.0
    inp = synth.randn_dense(1, 8, 1, 1, 70, d, d, dtype="bf16", sinks=True, seed=d + 2)
    dout = synth.randn_dout(1, 8, 1, d, seed=d + 2)
    check_bwd(inp, dout, causal=True, scale=1 / math.sqrt(d), label=f"d{d} Tq=1")


def test_bwd_deterministic_and_strided():
    """Two calls give identical bits; BSHD views (strided heads and tokens) give the same gradients."""
    announce("bwd determinism + strided")
    inp = synth.randn_dense(2, 8, 2, 150, 150, 128, 128, dtype="bf16", sinks=True, seed=11)
    dout = synth.randn_dout(2, 8, 150, 128, seed=11)
    a = run_fwd_bwd(inp, dout, causal=True, scale=0.09)
    b = run_fwd_bwd(inp, dout, causal=True, scale=0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # the same tensors as BSHD storage viewed as BHSD
    q, k, v = (inp[n].cuda().transpose(1, 2).contiguous().transpose(1, 2) for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda()
    out, lse = A.dense(q, k, v, causal=True, scale=0.09, sinks=sk)
    d = dout.cuda().transpose(1, 2).contiguous().transpose(1, 2)
    dq = torch.empty_like(q.transpose(1, 2).contiguous()).transpose(1, 2)
    r = A.dense_backward(q, k, v, out, d, lse, causal=True, scale=0.09, sinks=sk, dq=dq)
    torch.cuda.synchronize()
    for x, y in zip(a, r):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d,Hkv", [(512, 1), (256, 2)])
def test_bwd_wide_deterministic_and_strided(d, Hkv):
    """256/512-wide heads with the query heads split over workgroups (few key blocks):
    two calls give identical bits (the partials are added in a fixed order), and BSHD
    views with padded rows give the same gradients."""
    announce(f"bwd d{d} Hkv{Hkv} determinism + strided")
    B, H, T = 1, 16, 300
    inp = synth.randn_dense(B, H, Hkv, T, T, d, d, dtype="bf16", sinks=True, seed=d + Hkv)
    dout = synth.randn_dout(B, H, T, d, seed=d + Hkv)
    a = run_fwd_bwd(inp, dout, causal=True, scale=0.05)
    b = run_fwd_bwd(inp, dout, causal=True, scale=0.05)
    for x, y in zip(a, b):
        assert torch.equal(x, y)

    def bshd_padded(x):  # [B, N, T, d] -> a view of [B, T, N, d + 8] storage
        Bx, N, Tx, dx = x.shape
        store = torch.zeros(Bx, Tx, N, dx + 8, dtype=x.dtype, device="cuda")
        store[..., :dx] = x.cuda().transpose(1, 2)
        return store[..., :dx].transpose(1, 2)

    q, k, v = (bshd_padded(inp[n]) for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda()
    out, lse = A.dense(q, k, v, causal=True, scale=0.05, sinks=sk)
    r = A.dense_backward(q, k, v, out, bshd_padded(dout), lse, causal=True, scale=0.05, sinks=sk,
                         dq=bshd_padded(torch.zeros_like(inp["q"])), dk=bshd_padded(torch.zeros_like(inp["k"])),
                         dv=bshd_padded(torch.zeros_like(inp["v"])))
    torch.cuda.synchronize()
    for x, y in zip(a, r):
        assert torch.equal(x, y)


def test_bwd_rejects_bad_arguments():
    inp = synth.randn_dense(1, 4, 2, 8, 8, 128, 128, dtype="bf16", sinks=False, seed=1)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out, lse = A.dense(q, k, v, causal=True, scale=0.1)
    with pytest.raises(A.AttnInvalidArgument):   # dsinks without sinks
        A.dense_backward(q, k, v, out, out, lse, causal=True, scale=0.1,
                         dsinks=torch.empty(4, device="cuda"))
    with pytest.raises(A.AttnInvalidArgument):   # workspace too small
        A.dense_backward(q, k, v, out, out, lse, causal=True, scale=0.1,
                         workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    q5 = torch.zeros(1, 4, 8, 384, dtype=torch.bfloat16, device="cuda")
    k5 = torch.zeros(1, 2, 8, 384, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnUnsupported):       # head dims without a compiled backward
        A.dense_backward(q5, k5, k5, q5, q5, lse, causal=True, scale=0.1)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ full benchmark shapes, one kv group sampled
@pytest.mark.parametrize("wl,group", [(2, (1, 5)), (3, (3, 9)), (4, (0, 0))])
def test_bwd_full_workload_sampled_group(wl, group):
    """The benchmark's launch at full size; the oracle checks one (batch, kv head) group
    (every dq row of its heads, every dk/dv row of the kv head, the sink gradients of
    its heads): the gradient of a group depends on that group's inputs only. The
    512-wide MQA workload is one group of 64 heads whose dK/dV kernel splits the
    heads 16 ways."""
    s = synth.spec(wl)
    announce(f"bwd full workload {s.name} group {group}")
    inp = synth.make(wl)
    dout = synth.make_dout(s)
    dq, dk, dv, ds = run_fwd_bwd(inp, dout, causal=s.causal, scale=s.scale)
    b, kvh = group
    g = s.H // s.Hkv
    hs = slice(kvh * g, (kvh + 1) * g)
    sk = inp["sinks"][hs] if inp["sinks"] is not None else None
    rq, rk, rv, rs = oracle.dense_attention_backward(
        inp["q"][b:b + 1, hs], inp["k"][b:b + 1, kvh:kvh + 1], inp["v"][b:b + 1, kvh:kvh + 1], dout[b:b + 1, hs],
        scale=s.scale, causal=s.causal, sinks=sk)
    errs = {"dq": _rel_err(_np(dq[b:b + 1, hs]), rq), "dk": _rel_err(_np(dk[b:b + 1, kvh:kvh + 1]), rk),
            "dv": _rel_err(_np(dv[b:b + 1, kvh:kvh + 1]), rv)}
    assert max(errs.values()) <= TOL_REL, f"{s.name} group {group}: {errs}"
    if rs is not None and s.B == 1:      # dsinks sums over the batch: one batch is the whole sum
        es = _rel_err(_np(ds[hs]), rs)
        assert es <= TOL_SINK, f"{s.name}: dsinks rel err {es:.3e}"


def test_bwd_wide_many_key_blocks():
    """256-wide heads with 64 groups x 8 key blocks = 512 dK/dV workgroups: the heads of a
    group are not split (dk, dv written directly); two groups checked against the oracle."""
    announce("bwd d256 B64 H2/1 T512 (no head split)")
    B, H, Hkv, T, d = 64, 2, 1, 512, 256
    assert A.bwd_workspace_bytes(B, H, Hkv, T, T, d, d) == B * H * T * 4
    inp = synth.randn_dense(B, H, Hkv, T, T, d, d, dtype="bf16", sinks=True, seed=41)
    dout = synth.randn_dout(B, H, T, d, seed=41)
    dq, dk, dv, _ = run_fwd_bwd(inp, dout, causal=True, scale=1 / math.sqrt(d))
    for b in (0, B - 1):
        rq, rk, rv, _r = oracle.dense_attention_backward(
            inp["q"][b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1], dout[b:b + 1], scale=1 / math.sqrt(d),
            causal=True, sinks=inp["sinks"])
        errs = {"dq": _rel_err(_np(dq[b:b + 1]), rq), "dk": _rel_err(_np(dk[b:b + 1]), rk),
                "dv": _rel_err(_np(dv[b:b + 1]), rv)}
        assert max(errs.values()) <= TOL_REL, f"batch {b}: {errs}"


# ------------------------------------------------------------------ sliding windows
WIN_CASES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v, causal, sinks, window
    (1, 8, 2, 300, 300, 128, 128, True, True, (50, -1)),
    (1, 4, 2, 257, 257, 64, 64, False, False, (30, 90)),
    (1, 4, 4, 200, 333, 192, 128, True, False, (100, -1)),
    (2, 4, 1, 150, 150, 128, 128, True, False, (0, -1)),      # diagonal only
    (1, 8, 2, 100, 400, 128, 128, False, True, (-1, 20)),
    (1, 8, 1, 200, 200, 512, 512, True, True, (40, -1)),
    (1, 4, 2, 150, 260, 256, 256, False, False, (70, 25)),
]


@pytest.mark.parametrize("case", WIN_CASES, ids=lambda c: f"T{c[3]}x{c[4]}d{c[5]}w{c[9][0]}_{c[9][1]}"
                         f"{'c' if c[7] else 'n'}")
def test_bwd_window(case):
    B, H, Hkv, Tq, Tk, dqk, dv, causal, sinks, window = case
    announce(f"bwd window {case}")
    inp = synth.randn_dense(B, H, Hkv, Tq, Tk, dqk, dv, dtype="bf16", sinks=sinks, seed=Tq + 3 * Tk)
    dout = synth.randn_dout(B, H, Tq, dv, seed=Tq + 3 * Tk)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    scale = 1 / math.sqrt(dqk)
    out, lse = A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, window=window)
    dq, dk, dv_, ds = A.dense_backward(q, k, v, out, dout.cuda(), lse, causal=causal, scale=scale, sinks=sk,
                                       window=window)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.dense_attention_backward(inp["q"], inp["k"], inp["v"], dout, scale=scale, causal=causal,
                                                     sinks=inp["sinks"], window=window)
    errs = {"dq": _rel_err(_np(dq), rq), "dk": _rel_err(_np(dk), rk), "dv": _rel_err(_np(dv_), rv)}
    assert max(errs.values()) <= TOL_REL, f"{case}: {errs}"
    if rs is not None:
        assert _rel_err(_np(ds), rs) <= TOL_SINK


# ------------------------------------------------------------------ seeded random sweep
def _bwd_sweep_cases(n, seed):
    """Shapes drawn at random (seeded) over every compiled head-dim pair: GQA group
    (up to 16 heads a kv head, so the 256/512-wide kernels split heads), lengths
    with ragged tails, Tq != Tk, causal / sink / window switches."""
    rng = np.random.default_rng(seed)
    dims = [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)]
    cases = []
    for i in range(n):
        dqk, dv = dims[i % len(dims)]
        Hkv = int(rng.integers(1, 3))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        Tq = int(rng.integers(1, 260))
        Tk = Tq if rng.random() < 0.5 else int(rng.integers(1, 260))
        causal = bool(rng.random() < 0.7)
        win = (-1, -1)
        if rng.random() < 0.3:
            win = (int(rng.integers(0, 80)), -1 if causal else int(rng.integers(0, 80)))
        cases.append(dict(B=int(rng.integers(1, 3)), H=g * Hkv, Hkv=Hkv, Tq=Tq, Tk=Tk, dqk=dqk, dv=dv, causal=causal,
                          sinks=bool(rng.random() < 0.4), window=win, seed=2000 * seed + i))
    return cases


@pytest.mark.parametrize("case", _bwd_sweep_cases(15, 11), ids=lambda c: (
    f"B{c['B']}H{c['H']}/{c['Hkv']}T{c['Tq']}x{c['Tk']}d{c['dqk']}/{c['dv']}"
    f"{'c' if c['causal'] else 'n'}{'s' if c['sinks'] else ''}w{c['window'][0]}_{c['window'][1]}"))
def test_bwd_random_sweep(case):
    c = case
    announce(f"bwd sweep {c}")
    inp = synth.randn_dense(c["B"], c["H"], c["Hkv"], c["Tq"], c["Tk"], c["dqk"], c["dv"], dtype="bf16",
                            sinks=c["sinks"], seed=c["seed"])
    dout = synth.randn_dout(c["B"], c["H"], c["Tq"], c["dv"], seed=c["seed"])
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    scale = 1 / math.sqrt(c["dqk"])
    out, lse = A.dense(q, k, v, causal=c["causal"], scale=scale, sinks=sk, window=c["window"])
    dq, dk, dv_, ds = A.dense_backward(q, k, v, out, dout.cuda(), lse, causal=c["causal"], scale=scale, sinks=sk,
                                       window=c["window"])
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.dense_attention_backward(inp["q"], inp["k"], inp["v"], dout, scale=scale,
                                                     causal=c["causal"], sinks=inp["sinks"], window=c["window"])
    errs = {"dq": _rel_err(_np(dq), rq), "dk": _rel_err(_np(dk), rk), "dv": _rel_err(_np(dv_), rv)}
    assert max(errs.values()) <= TOL_REL, f"{c}: {errs}"
    if rs is not None:
        assert _rel_err(_np(ds), rs) <= TOL_SINK, f"{c}: dsinks"
