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


def check_bwd_dropout(orc=oracle):
    """Dropout in the backward: central differences of the forward with the same mask
    (the forward and the backward share it), and torch autograd through an explicit
    mask multiply."""
    worst = 0.0
    rng = np.random.default_rng(995)
    B, H, Hkv, Tq, Tk, dqk, dv = 1, 4, 2, 6, 7, 4, 3
    q, k, v = _rand((B, H, Tq, dqk), 996, 0.8), _rand((B, Hkv, Tk, dqk), 997, 0.8), _rand((B, Hkv, Tk, dv), 998)
    G = _rand((B, H, Tq, dv), 999)
    sinks = _rand((H,), 1000)
    keep = rng.random((B, H, Tq, Tk)) > 0.35
    for causal in (False, True):
        sk = sinks.copy()
        gq, gk, gv, gs = orc.dense_attention_backward(q, k, v, G, scale=0.5, causal=causal, sinks=sk, keep=keep,
                                                      p_drop=0.35)

        def f():
            o, _ = orc.dense_attention(q, k, v, scale=0.5, causal=causal, sinks=sk, keep=keep, p_drop=0.35)
            return float((o * G).sum())
        worst = max(worst, _err(gq, _fd_grad(f, q)) / TOL_FD * TOL, _err(gk, _fd_grad(f, k)) / TOL_FD * TOL,
                    _err(gv, _fd_grad(f, v)) / TOL_FD * TOL, _err(gs, _fd_grad(f, sk)) / TOL_FD * TOL)
        Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        g = H // Hkv
        s = torch.matmul(Q, K.repeat_interleave(g, dim=1).transpose(-1, -2)) * 0.5
        if causal:
            s = s.masked_fill(~torch.ones(Tq, Tk, dtype=torch.bool).tril(diagonal=Tk - Tq), float("-inf"))
        p = torch.softmax(s, dim=-1) * torch.from_numpy(keep) / 0.65
        (torch.matmul(p, V.repeat_interleave(g, dim=1)) * torch.from_numpy(G)).sum().backward()
        gq, gk, gv, _ = orc.dense_attention_backward(q, k, v, G, scale=0.5, causal=causal, keep=keep, p_drop=0.35)
        worst = max(worst, _err(gq, Q.grad.numpy()), _err(gk, K.grad.numpy()), _err(gv, V.grad.numpy()))
    return worst


def _sparse_loss(orc, q, kv, idx, G, d_v, scale, sinks):
    o, _ = orc.sparse_topk_attention(q, kv, idx, d_v=d_v, scale=scale, sinks=sinks)
    return float((o * G).sum())


SPARSE_IDX = np.array([[0, 3, 3, 5], [6, 1, -1, 2], [4, 4, 4, 0]])   # duplicates and a skipped slot


def check_sparse_bwd_finite_differences(orc=oracle):
    """dq, dkv, dsinks of the sparse forward against central differences: duplicated
    indices, a skipped (-1) slot, V the first d_v < d_qk columns of the pool."""
    worst = 0.0
    Sq, Hq, N, dqk, dv = 3, 2, 7, 5, 3
    q = _rand((Sq, Hq, dqk), 360, 0.8)
    kv = _rand((N, dqk), 361, 0.8)
    G = _rand((Sq, Hq, dv), 362)
    sinks = _rand((Hq,), 363)
    for sk in (None, sinks.copy()):
        gq, gkv, gs = orc.sparse_topk_attention_backward(q, kv, SPARSE_IDX, G, d_v=dv, scale=0.6, sinks=sk)
        f = lambda: _sparse_loss(orc, q, kv, SPARSE_IDX, G, dv, 0.6, sk)  # noqa: E731
        worst = max(worst, _err(gq, _fd_grad(f, q)), _err(gkv, _fd_grad(f, kv)))
        if sk is not None:
            worst = max(worst, _err(gs, _fd_grad(f, sk)))
    return worst / TOL_FD * TOL


def check_sparse_bwd_library_autograd(orc=oracle):
    """torch autograd (fp64) through index_select + softmax with an explicit sink column."""
    worst = 0.0
    Sq, Hq, N, d, topk = 4, 3, 9, 6, 5
    q, kv = _rand((Sq, Hq, d), 370), _rand((N, d), 371)
    rng = np.random.default_rng(372)
    idx = np.stack([rng.choice(N, topk, replace=False) for _ in range(Sq)])
    G = _rand((Sq, Hq, d), 373)
    sinks = _rand((Hq,), 374)
    for sk in (None, sinks):
        Q, KV = torch.tensor(q, requires_grad=True), torch.tensor(kv, requires_grad=True)
        S_ = torch.tensor(sk, requires_grad=True) if sk is not None else None
        outs = []
        for s in range(Sq):
            g = KV.index_select(0, torch.from_numpy(idx[s]))
            sc = 0.45 * Q[s] @ g.T
            if S_ is not None:
                p = torch.softmax(torch.cat([sc, S_[:, None]], dim=1), dim=1)[:, :topk]
            else:
                p = torch.softmax(sc, dim=1)
            outs.append(p @ g)
        (torch.stack(outs) * torch.from_numpy(G)).sum().backward()
        gq, gkv, gs = orc.sparse_topk_attention_backward(q, kv, idx, G, d_v=d, scale=0.45, sinks=sk)
        worst = max(worst, _err(gq, Q.grad.numpy()), _err(gkv, KV.grad.numpy()))
        if sk is not None:
            worst = max(worst, _err(gs, S_.grad.numpy()))
    return worst


def check_sparse_bwd_equals_dense_mqa(orc=oracle):
    """Every query naming the whole pool (d_v = d_qk) is dense non-causal MQA with k = v =
    the pool: dq equal, and the pool's gradient is the dense dk + dv."""
    Sq, Hq, N, d = 5, 4, 6, 4
    q, kv, G = _rand((Sq, Hq, d), 380), _rand((N, d), 381), _rand((Sq, Hq, d), 382)
    sinks = _rand((Hq,), 383)
    idx = np.tile(np.arange(N), (Sq, 1))
    gq, gkv, gs = orc.sparse_topk_attention_backward(q, kv, idx, G, d_v=d, scale=0.5, sinks=sinks)
    dq, dk, dv, ds = orc.dense_attention_backward(q.transpose(1, 0, 2)[None], kv[None, None], kv[None, None],
                                                  G.transpose(1, 0, 2)[None], scale=0.5, causal=False, sinks=sinks)
    return max(_err(gq, dq[0].transpose(1, 0, 2)), _err(gkv, dk[0, 0] + dv[0, 0]), _err(gs, ds))


ALL_CHECKS = {
    "bwd_dropout": check_bwd_dropout,
    "sparse_bwd_finite_differences": check_sparse_bwd_finite_differences,
    "sparse_bwd_library_autograd": check_sparse_bwd_library_autograd,
    "sparse_bwd_equals_dense_mqa": check_sparse_bwd_equals_dense_mqa,
    "bwd_window_finite_differences": check_bwd_window_finite_differences,
    "bwd_finite_differences": check_bwd_finite_differences,
    "bwd_library_autograd": check_bwd_library_autograd,
    "bwd_invariants": check_bwd_invariants,
    "bwd_closed_forms": check_bwd_closed_forms,
    "bwd_sink_limit": check_bwd_sink_limit,
    "bwd_masked_rows": check_bwd_masked_rows,
}
