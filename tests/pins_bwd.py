"""Checks that pin the oracle's backward to things other than itself.

Each ``check_*`` returns the largest discrepancy it found (0 means "holds").
Sources of truth: central finite differences of the oracle's forward (which
is pinned on its own by tests/pins.py), torch autograd in fp64 through an
explicitly written softmax (a library's chain rule, not the oracle's),
closed forms and invariants of the gradient.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from tests.pins import _err, _rand

TOL = 1e-10      # exact comparisons (library autograd, closed forms, invariants)
TOL_FD = 1e-7    # central differences with h = 1e-5 in fp64


def _loss(orc, q, k, v, sinks, G, scale, causal, window=(-1, -1)):
    o, _ = orc.dense_attention(q, k, v, scale=scale, causal=causal, sinks=sinks, window=window)
    return float((o * G).sum())


def _fd_grad(f, x, h=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        up = f()
        x[i] = old - h
        dn = f()
        x[i] = old
        g[i] = (up - dn) / (2 * h)
    return g


FD_SHAPES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v
    (1, 4, 2, 5, 7, 6, 5),
    (1, 2, 1, 6, 4, 3, 4),     # Tq > Tk: early rows see no key under causal
    (2, 3, 3, 3, 3, 4, 2),
]


def check_bwd_finite_differences(orc=oracle):
    """dL/dq, dL/dk, dL/dv, dL/dsinks for L = sum(O * G), against central differences."""
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, dqk, dv) in enumerate(FD_SHAPES):
        q = _rand((B, H, Tq, dqk), 300 + i, 0.8)
        k = _rand((B, Hkv, Tk, dqk), 310 + i, 0.8)
        v = _rand((B, Hkv, Tk, dv), 320 + i)
        G = _rand((B, H, Tq, dv), 330 + i)
        sinks = _rand((H,), 340 + i)
        scale = 1.0 / math.sqrt(dqk)
        for causal in (False, True):
            for sk in (None, sinks.copy()):
                gq, gk, gv, gs = orc.dense_attention_backward(q, k, v, G, scale=scale, causal=causal, sinks=sk)
                f = lambda: _loss(orc, q, k, v, sk, G, scale, causal)  # noqa: E731
                worst = max(worst, _err(gq, _fd_grad(f, q)), _err(gk, _fd_grad(f, k)), _err(gv, _fd_grad(f, v)))
                if sk is not None:
                    worst = max(worst, _err(gs, _fd_grad(f, sk)))
    return worst / TOL_FD * TOL  # reported on the TOL scale


def _torch_attention(Q, K, V, sinks, scale, causal):
    """Attention written with torch ops (fp64); autograd supplies the gradients."""
    g = Q.shape[1] // K.shape[1]
    Kr = K.repeat_interleave(g, dim=1)
    Vr = V.repeat_interleave(g, dim=1)
    Tq, Tk = Q.shape[2], K.shape[2]
    s = torch.matmul(Q, Kr.transpose(-1, -2)) * scale
    if causal:
        mask = torch.ones(Tq, Tk, dtype=torch.bool).tril(diagonal=Tk - Tq)
        s = s.masked_fill(~mask, float("-inf"))
    if sinks is not None:
        col = sinks.view(1, -1, 1, 1).expand(s.shape[0], -1, Tq, 1)
        p = torch.softmax(torch.cat([s, col], dim=-1), dim=-1)[..., :Tk]
    else:
        p = torch.softmax(s, dim=-1)
    return torch.matmul(p, Vr)


def check_bwd_library_autograd(orc=oracle):
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, dqk, dv) in enumerate([(2, 8, 2, 33, 33, 16, 16), (1, 4, 1, 20, 45, 8, 12),
                                                       (1, 6, 3, 40, 40, 24, 8)]):
        q, k, v = _rand((B, H, Tq, dqk), 400 + i), _rand((B, Hkv, Tk, dqk), 410 + i), _rand((B, Hkv, Tk, dv), 420 + i)
        G = _rand((B, H, Tq, dv), 430 + i)
        sinks = _rand((H,), 440 + i)
        for causal in (False, True):
            for sk in (None, sinks):
                Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
                S = torch.tensor(sk, requires_grad=True) if sk is not None else None
                out = _torch_attention(Q, K, V, S, 0.3, causal)
                (out * torch.from_numpy(G)).sum().backward()
                gq, gk, gv, gs = orc.dense_attention_backward(q, k, v, G, scale=0.3, causal=causal, sinks=sk)
                worst = max(worst, _err(gq, Q.grad.numpy()), _err(gk, K.grad.numpy()), _err(gv, V.grad.numpy()))
                if sk is not None:
                    worst = max(worst, _err(gs, S.grad.numpy()))
    return worst


def check_bwd_invariants(orc=oracle):
    """Without sinks and with every row seeing a key: each row of dS sums to 0, so the
    keys' gradients of one kv head sum to 0, and the values' gradients sum to the rows' dO."""
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, d) in enumerate([(1, 4, 2, 9, 9, 8), (2, 6, 1, 5, 11, 4)]):
        q, k, v = _rand((B, H, Tq, d), 500 + i), _rand((B, Hkv, Tk, d), 510 + i), _rand((B, Hkv, Tk, d), 520 + i)
        G = _rand((B, H, Tq, d), 530 + i)
        for causal in (False, True):
            gq, gk, gv, _ = orc.dense_attention_backward(q, k, v, G, scale=0.5, causal=causal)
            worst = max(worst, _err(gk.sum(axis=2), 0.0))
            dO_sum = oracle.sum_kv_groups(G, H // Hkv).sum(axis=2)
            worst = max(worst, _err(gv.sum(axis=2), dO_sum))
    return worst


def check_bwd_closed_forms(orc=oracle):
    """One visible key and no sink: P = 1, so dS = 0 (dq = dk = 0) and dv = the summed dO.
    Uniform scores (k = 0): P = 1/n, O = mean(v), and dv_j = dO / n for every key."""
    worst = 0.0
    q, k, v = _rand((1, 2, 4, 3), 600), _rand((1, 1, 1, 3), 601), _rand((1, 1, 1, 5), 602)
    G = _rand((1, 2, 4, 5), 603)
    gq, gk, gv, _ = orc.dense_attention_backward(q, k, v, G, scale=0.7, causal=False)
    worst = max(worst, _err(gq, 0.0), _err(gk, 0.0), _err(gv[0, 0, 0], G[0].sum(axis=(0, 1))))
    n = 6
    q, v = _rand((1, 1, 3, 4), 604), _rand((1, 1, n, 2), 605)
    k = np.zeros((1, 1, n, 4))
    G = _rand((1, 1, 3, 2), 606)
    gq, gk, gv, _ = orc.dense_attention_backward(q, k, v, G, scale=1.0, causal=False)
    worst = max(worst, _err(gv[0, 0], np.repeat(G[0, 0].sum(axis=0, keepdims=True) / n, n, axis=0)))
    # dq with uniform P: scale * sum_j P_j (dP_j - D) k_j = 0 because k = 0
    worst = max(worst, _err(gq, 0.0))
    return worst


def check_bwd_sink_limit(orc=oracle):
    """A sink of -inf is no sink: same gradients, and its own gradient is 0."""
    q, k, v = _rand((1, 4, 6, 5), 700), _rand((1, 2, 6, 5), 701), _rand((1, 2, 6, 3), 702)
    G = _rand((1, 4, 6, 3), 703)
    a = orc.dense_attention_backward(q, k, v, G, scale=0.4, causal=True)
    b = orc.dense_attention_backward(q, k, v, G, scale=0.4, causal=True, sinks=np.full(4, -np.inf))
    return max(_err(a[0], b[0]), _err(a[1], b[1]), _err(a[2], b[2]), _err(b[3], 0.0))


def check_bwd_masked_rows(orc=oracle):
    """Tq > Tk, causal: rows that see no key have zero dq and give nothing to dk, dv."""
    q, k, v = _rand((1, 2, 7, 4), 800), _rand((1, 1, 3, 4), 801), _rand((1, 1, 3, 2), 802)
    G = _rand((1, 2, 7, 2), 803)
    gq, gk, gv, _ = orc.dense_attention_backward(q, k, v, G, scale=0.5, causal=True)
    G2 = G.copy()
    G2[:, :, :4] = 123.0          # rows 0..3 see no key (key j visible iff j <= t - 4)
    gq2, gk2, gv2, _ = orc.dense_attention_backward(q, k, v, G2, scale=0.5, causal=True)
    return max(_err(gq[:, :, :4], 0.0), _err(gk, gk2), _err(gv, gv2))


def check_bwd_window_finite_differences(orc=oracle):
    """Sliding windows: the gradients against central differences of the windowed forward."""
    worst = 0.0
    B, H, Hkv, Tq, Tk, dqk, dv = 1, 4, 2, 7, 9, 4, 3
    q = _rand((B, H, Tq, dqk), 350, 0.8)
    k = _rand((B, Hkv, Tk, dqk), 351, 0.8)
    v = _rand((B, Hkv, Tk, dv), 352)
    G = _rand((B, H, Tq, dv), 353)
    sinks = _rand((H,), 354)
    for causal, win in ((True, (2, -1)), (False, (1, 2)), (True, (0, -1))):
        sk = sinks.copy()
        gq, gk, gv, gs = orc.dense_attention_backward(q, k, v, G, scale=0.5, causal=causal, sinks=sk, window=win)
        f = lambda: _loss(orc, q, k, v, sk, G, 0.5, causal, win)  # noqa: E731
        worst = max(worst, _err(gq, _fd_grad(f, q)), _err(gk, _fd_grad(f, k)), _err(gv, _fd_grad(f, v)),
                    _err(gs, _fd_grad(f, sk)))
    return worst / TOL_FD * TOL


ALL_CHECKS = {
    "bwd_window_finite_differences": check_bwd_window_finite_differences,
    "bwd_finite_differences": check_bwd_finite_differences,
    "bwd_library_autograd": check_bwd_library_autograd,
    "bwd_invariants": check_bwd_invariants,
    "bwd_closed_forms": check_bwd_closed_forms,
    "bwd_sink_limit": check_bwd_sink_limit,
    "bwd_masked_rows": check_bwd_masked_rows,
}
