"""Checks that pin the fp64 oracle to things other than itself.

Each ``check_*`` returns the largest discrepancy it found (0 means "holds").
The pin tests assert every check is within tolerance; the mutation tests plant
a mistake in the oracle and assert that some check fails.

Sources of truth used here: brute force (tests/brute.py, a different
formulation in pure Python), library routines (torch's scaled_dot_product_attention
in fp64, scipy's logsumexp), closed forms, and invariants of the definition.
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp

import oracle
from oracle import attention as OA
from tests.brute import brute_dense, brute_extras, brute_sparse, brute_two_part

TOL = 1e-12


def _err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force
BRUTE_SHAPES = [
    # B, H, Hkv, Tq, Tk, d_qk, d_v
    (1, 1, 1, 1, 1, 1, 1),
    (1, 2, 1, 3, 3, 3, 2),
    (1, 4, 2, 5, 5, 8, 3),
    (2, 4, 1, 5, 7, 3, 8),
    (1, 2, 2, 7, 4, 8, 8),     # Tq > Tk: early rows fully masked under causal
    (1, 4, 4, 17, 17, 3, 1),
]


def check_brute_dense(orc=oracle, shapes=BRUTE_SHAPES):
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, dqk, dv) in enumerate(shapes):
        q = _rand((B, H, Tq, dqk), 10 + i, 0.7)
        k = _rand((B, Hkv, Tk, dqk), 20 + i, 0.7)
        v = _rand((B, Hkv, Tk, dv), 30 + i)
        sinks = _rand((H,), 40 + i)
        for causal in (False, True):
            for sk in (None, sinks):
                scale = 1.0 / math.sqrt(dqk)
                o, l = orc.dense_attention(q, k, v, scale=scale, causal=causal, sinks=sk)
                bo, bl = brute_dense(q, k, v, scale, causal, sk)
                worst = max(worst, _err(o, bo), _err(l, bl))
    return worst


def check_brute_sparse(orc=oracle):
    worst = 0.0
    for i, (Sq, Hq, N, dqk, dv, topk) in enumerate([(1, 1, 4, 2, 2, 2), (3, 4, 9, 5, 3, 4),
                                                      (2, 2, 6, 8, 8, 6)]):
        q = _rand((Sq, Hq, dqk), 50 + i, 0.7)
        kv = _rand((N, dqk), 60 + i)
        rng = np.random.default_rng(70 + i)
        idx = np.stack([rng.choice(N, topk, replace=False) for _ in range(Sq)]).astype(np.int32)
        idx[0, 0] = -1                      # one skipped entry
        sinks = _rand((Hq,), 80 + i)
        for sk in (None, sinks):
            o, l = orc.sparse_topk_attention(q, kv, idx, d_v=dv, scale=0.4, sinks=sk)
            bo, bl = brute_sparse(q, kv, idx, dv, 0.4, sk)
            worst = max(worst, _err(o, bo), _err(l, bl))
    return worst


# ---------------------------------------------------------------- library routines
def _torch_reference(q, k, v, scale, causal):
    """torch SDPA (math path, CPU fp64), GQA by torch's own repeat_interleave."""
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    g = Q.shape[1] // K.shape[1]
    K = K.repeat_interleave(g, dim=1).contiguous()
    V = V.repeat_interleave(g, dim=1).contiguous()
    Tq, Tk = Q.shape[2], K.shape[2]
    mask = None
    if causal:  # bottom-right aligned boolean mask
        mask = torch.ones(Tq, Tk, dtype=torch.bool).tril(diagonal=Tk - Tq)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), logsumexp(s.numpy(), axis=-1)


def check_library_dense(orc=oracle):
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, d) in enumerate([(2, 8, 2, 33, 33, 16), (1, 4, 1, 20, 45, 8),
                                                 (1, 6, 3, 64, 64, 32)]):
        q, k, v = _rand((B, H, Tq, d), 90 + i), _rand((B, Hkv, Tk, d), 91 + i), _rand((B, Hkv, Tk, d), 92 + i)
        for causal in (False, True):
            o, l = orc.dense_attention(q, k, v, scale=0.3, causal=causal)
            to, tl = _torch_reference(q, k, v, 0.3, causal)
            worst = max(worst, _err(o, to), _err(l, tl))
    return worst


# ---------------------------------------------------------------- closed forms
def check_closed_forms(orc=oracle):
    worst = 0.0
    B, H, Hkv, T, d = 1, 4, 2, 9, 5
    q, k, v = _rand((B, H, T, d), 1), _rand((B, Hkv, T, d), 2), _rand((B, Hkv, T, d), 3)
    scale = 0.45
    o, l = orc.dense_attention(q, k, v, scale=scale, causal=True)
    g = H // Hkv
    for h in range(H):
        # causal row 0 sees only key 0: O = v_0, lse = scale * q_0 . k_0
        worst = max(worst, _err(o[0, h, 0], v[0, h // g, 0]))
        worst = max(worst, _err(l[0, h, 0], scale * float(q[0, h, 0] @ k[0, h // g, 0])))
    # the last causal row equals the non-causal result for that row
    onc, lnc = orc.dense_attention(q, k, v, scale=scale, causal=False)
    worst = max(worst, _err(o[:, :, -1], onc[:, :, -1]), _err(l[:, :, -1], lnc[:, :, -1]))
    # uniform scores (q = 0): O = mean of the visible V rows, lse = ln n
    qz = np.zeros_like(q)
    oz, lz = orc.dense_attention(qz, k, v, scale=scale, causal=True)
    sinks = _rand((H,), 4)
    ozs, lzs = orc.dense_attention(qz, k, v, scale=scale, causal=True, sinks=sinks)
    for h in range(H):
        for t in range(T):
            n = t + 1
            mean = v[0, h // g, :n].mean(axis=0)
            worst = max(worst, _err(oz[0, h, t], mean), _err(lz[0, h, t], math.log(n)))
            # with a sink: O = n / (n + e^s) * mean, lse = ln(n + e^s)
            es = math.exp(sinks[h])
            worst = max(worst, _err(ozs[0, h, t], n / (n + es) * mean),
                        _err(lzs[0, h, t], math.log(n + es)))
    # two keys: weights are the logistic function of the score difference
    q2, k2, v2 = _rand((1, 1, 1, 3), 5), _rand((1, 1, 2, 3), 6), _rand((1, 1, 2, 4), 7)
    o2, l2 = orc.dense_attention(q2, k2, v2, scale=1.0, causal=False)
    sa, sb = float(q2[0, 0, 0] @ k2[0, 0, 0]), float(q2[0, 0, 0] @ k2[0, 0, 1])
    wa = 1.0 / (1.0 + math.exp(sb - sa))
    worst = max(worst, _err(o2[0, 0, 0], wa * v2[0, 0, 0] + (1 - wa) * v2[0, 0, 1]))
    worst = max(worst, _err(l2[0, 0, 0], max(sa, sb) + math.log1p(math.exp(-abs(sa - sb)))))
    return worst


def check_window(orc=oracle):
    """Sliding windows: brute force (different formulation), the diagonal-only
    closed form, wide windows equal no window, and a window never widens causal."""
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, d) in enumerate([(1, 4, 2, 9, 9, 5), (2, 2, 1, 5, 11, 3), (1, 2, 2, 8, 4, 4)]):
        q = _rand((B, H, Tq, d), 700 + i, 0.7)
        k = _rand((B, Hkv, Tk, d), 710 + i, 0.7)
        v = _rand((B, Hkv, Tk, d), 720 + i)
        sinks = _rand((H,), 730 + i)
        for causal in (False, True):
            for win in ((0, -1), (2, -1), (3, 1), (-1, 2), (1, 0), (0, 0)):
                for sk in (None, sinks):
                    o, l = orc.dense_attention(q, k, v, scale=0.5, causal=causal, sinks=sk, window=win)
                    bo, bl = brute_dense(q, k, v, 0.5, causal, sk, window=win)
                    worst = max(worst, _err(o, bo), _err(l, bl))
    # left = 0 with causal: each row sees only its diagonal key (Tq = Tk)
    q, k, v = _rand((1, 2, 6, 4), 740), _rand((1, 1, 6, 4), 741), _rand((1, 1, 6, 3), 742)
    o, l = orc.dense_attention(q, k, v, scale=0.5, causal=True, window=(0, -1))
    for h in range(2):
        for t in range(6):
            worst = max(worst, _err(o[0, h, t], v[0, 0, t]), _err(l[0, h, t], 0.5 * float(q[0, h, t] @ k[0, 0, t])))
    # windows wider than the keys are no window; with causal, any right bound is causal
    for causal in (False, True):
        base = orc.dense_attention(q, k, v, scale=0.5, causal=causal)
        wide = orc.dense_attention(q, k, v, scale=0.5, causal=causal, window=(6, 6))
        worst = max(worst, _err(base[0], wide[0]), _err(base[1], wide[1]))
    c = orc.dense_attention(q, k, v, scale=0.5, causal=True)
    cw = orc.dense_attention(q, k, v, scale=0.5, causal=True, window=(-1, 3))
    worst = max(worst, _err(c[0], cw[0]), _err(c[1], cw[1]))
    return worst


def check_varlen(orc=oracle):
    """Packed sequences: equal lengths give the padded batch exactly; ragged lengths
    (including an empty sequence and Tq != Tk) match brute force per sequence; and a
    sequence's output ignores every other sequence's keys."""
    worst = 0.0
    B, H, Hkv, T, d = 3, 4, 2, 6, 5
    q, k, v = _rand((B, H, T, d), 900), _rand((B, Hkv, T, d), 901), _rand((B, Hkv, T, 3), 902)
    sinks = _rand((H,), 903)
    cu = np.arange(B + 1) * T
    pack = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(-1, x.shape[1], x.shape[3]))  # noqa: E731
    for causal in (False, True):
        o, l = orc.dense_attention(q, k, v, scale=0.4, causal=causal, sinks=sinks)
        ov, lv = orc.dense_attention_varlen(pack(q), pack(k), pack(v), cu, cu, scale=0.4, causal=causal, sinks=sinks)
        worst = max(worst, _err(ov, pack(o)), _err(lv, l.transpose(1, 0, 2).reshape(H, -1)))
    lq, lk = [3, 0, 7, 1], [5, 2, 4, 1]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = _rand((cq[-1], H, d), 904)
    k, v = _rand((ck[-1], Hkv, d), 905), _rand((ck[-1], Hkv, 3), 906)
    for causal in (False, True):
        for win in ((-1, -1), (1, -1)):
            ov, lv = orc.dense_attention_varlen(q, k, v, cq, ck, scale=0.4, causal=causal, sinks=sinks, window=win)
            for b in range(len(lq)):
                if lq[b] == 0:
                    continue
                qb = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
                kb = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
                vb = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
                bo, bl = brute_dense(qb, kb, vb, 0.4, causal, sinks, window=win)
                worst = max(worst, _err(ov[cq[b]:cq[b + 1]], np.asarray(bo)[0].transpose(1, 0, 2)),
                            _err(lv[:, cq[b]:cq[b + 1]], np.asarray(bl)[0]))
            # isolation: scrambling sequence 3's keys leaves the others unchanged
            k2 = k.copy()
            k2[ck[3]:ck[4]] += 10.0
            ov2, lv2 = orc.dense_attention_varlen(q, k2, v, cq, ck, scale=0.4, causal=causal, sinks=sinks, window=win)
            worst = max(worst, _err(ov2[:cq[3]], ov[:cq[3]]), _err(lv2[:, :cq[3]], lv[:, :cq[3]]))
    return worst


def check_causal_differs(orc=oracle):
    """Causal must not silently equal full attention (returns 0 when it differs)."""
    q, k, v = _rand((1, 2, 8, 4), 11), _rand((1, 1, 8, 4), 12), _rand((1, 1, 8, 4), 13)
    o, _ = orc.dense_attention(q, k, v, scale=0.5, causal=True)
    onc, _ = orc.dense_attention(q, k, v, scale=0.5, causal=False)
    diff = np.abs(o[:, :, :-1] - onc[:, :, :-1]).max()
    return 0.0 if diff > 1e-3 else 1.0


def check_fully_masked_rows(orc=oracle):
    """Tq > Tk with a bottom-right causal mask: the first Tq - Tk rows see nothing."""
    q, k, v = _rand((1, 2, 6, 3), 14), _rand((1, 1, 2, 3), 15), _rand((1, 1, 2, 3), 16)
    sinks = np.array([0.3, -1.2])
    o, l = orc.dense_attention(q, k, v, scale=0.5, causal=True)
    os_, ls = orc.dense_attention(q, k, v, scale=0.5, causal=True, sinks=sinks)
    worst = max(_err(o[0, :, :4], 0.0), _err(os_[0, :, :4], 0.0))
    worst = max(worst, _err(l[0, :, :4], -np.inf))
    for h in range(2):
        worst = max(worst, _err(ls[0, h, :4], sinks[h]))
    return worst


# ---------------------------------------------------------------- invariants
def check_fold_matches_repeat_kv(orc=oracle):
    """The folded (reshape) computation equals the repeat_kv computation."""
    worst = 0.0
    for g in (1, 2, 4, 8, 64):
        Hkv = 2 if g < 64 else 1
        H = g * Hkv
        q, k, v = _rand((1, H, 6, 4), 100 + g), _rand((1, Hkv, 6, 4), 200 + g), _rand((1, Hkv, 6, 3), 300 + g)
        sinks = _rand((H,), 400 + g)
        a = orc.dense_attention(q, k, v, scale=0.5, causal=True, sinks=sinks)
        b = orc.dense_attention_tiled(q, k, v, scale=0.5, causal=True, sinks=sinks,
                                      tile_bytes=1 << 30)
        worst = max(worst, _err(a[0], b[0]), _err(a[1], b[1]))
        # and both equal brute force, whose head mapping is kv = h // g
        bo, bl = brute_dense(q, k, v, 0.5, True, sinks)
        worst = max(worst, _err(a[0], bo), _err(a[1], bl))
    return worst


def check_tiling_exact(orc=oracle):
    """Row tiling is exact and the mask follows the tile, with head-straddling tiles."""
    worst = 0.0
    B, H, Hkv, T, d = 1, 8, 1, 13, 4
    q, k, v = _rand((B, H, T, d), 21), _rand((B, Hkv, T, d), 22), _rand((B, Hkv, T, d), 23)
    sinks = _rand((H,), 24)
    full = orc.dense_attention(q, k, v, scale=0.5, causal=True, sinks=sinks)
    for rows in (1, 5, 13, 17, 40, 104):
        tb = rows * T * 8
        straddles = (rows % T) != 0
        tiled = orc.dense_attention_tiled(q, k, v, scale=0.5, causal=True, sinks=sinks, tile_bytes=tb)
        worst = max(worst, _err(full[0], tiled[0]), _err(full[1], tiled[1]))
        if rows in (5, 17, 40):
            assert straddles
    return worst


def check_sink_limit(orc=oracle):
    """A sink of -inf is no sink; a very negative sink tends to no sink."""
    q, k, v = _rand((1, 4, 7, 5), 31), _rand((1, 2, 7, 5), 32), _rand((1, 2, 7, 3), 33)
    base = orc.dense_attention(q, k, v, scale=0.5, causal=True)
    inf = orc.dense_attention(q, k, v, scale=0.5, causal=True, sinks=np.full(4, -np.inf))
    return max(_err(base[0], inf[0]), _err(base[1], inf[1]))


def check_shift_invariance(orc=oracle):
    """Adding c to every score and to the sink leaves O and shifts lse by c.

    The shift is applied through an extra feature: q' = [q, c/scale], k' = [k, 1].
    """
    c, scale = 0.8, 0.5
    q, k, v = _rand((1, 2, 6, 4), 41), _rand((1, 1, 6, 4), 42), _rand((1, 1, 6, 3), 43)
    sinks = _rand((2,), 44)
    a = orc.dense_attention(q, k, v, scale=scale, causal=True, sinks=sinks)
    q2 = np.concatenate([q, np.full(q.shape[:-1] + (1,), c / scale)], axis=-1)
    k2 = np.concatenate([k, np.ones(k.shape[:-1] + (1,))], axis=-1)
    b = orc.dense_attention(q2, k2, v, scale=scale, causal=True, sinks=sinks + c)
    return max(_err(a[0], b[0]), _err(a[1] + c, b[1]))


def check_kv_split_merge(orc=oracle):
    """(O, lse) over disjoint key sets merge to the full result (sink counted once)."""
    Sq, Hq, N, d = 3, 4, 12, 6
    q, kv = _rand((Sq, Hq, d), 51), _rand((N, d), 52)
    sinks = _rand((Hq,), 53)
    idx = np.tile(np.arange(N, dtype=np.int32), (Sq, 1))
    full = orc.sparse_topk_attention(q, kv, idx, d_v=d, scale=0.4, sinks=sinks)
    pa = orc.sparse_topk_attention(q, kv, idx[:, :5], d_v=d, scale=0.4)
    pb = orc.sparse_topk_attention(q, kv, idx[:, 5:], d_v=d, scale=0.4)
    worst = 0.0
    for h in range(Hq):
        mo, ml = orc.merge_partials([(pa[0][:, h], pa[1][:, h]), (pb[0][:, h], pb[1][:, h])],
                                    sink=float(sinks[h]))
        worst = max(worst, _err(mo, full[0][:, h]), _err(ml, full[1][:, h]))
    return worst


def check_sparse_equals_dense_mqa(orc=oracle):
    """All of [0, N) as the index list = dense non-causal MQA over the pool (V == K)."""
    Sq, Hq, N, d = 5, 4, 9, 6
    q, kv = _rand((Sq, Hq, d), 61), _rand((N, d), 62)
    rng = np.random.default_rng(63)
    idx = np.stack([rng.permutation(N) for _ in range(Sq)]).astype(np.int32)
    so, sl = orc.sparse_topk_attention(q, kv, idx, d_v=d, scale=0.4)
    # dense: heads as H, one kv head, queries as tokens, keys = the pool in order
    qd = q.transpose(1, 0, 2)[None]                     # [1, Hq, Sq, d]
    kd = kv[None, None]                                 # [1, 1, N, d]
    do, dl = orc.dense_attention(qd, kd, kd, scale=0.4, causal=False)
    return max(_err(so, do[0].transpose(1, 0, 2)), _err(sl, dl[0].T))


def check_sparse_conventions(orc=oracle):
    """Permutation invariance, duplicate = +ln 2, -1 skipped, gather = one-hot product."""
    Sq, Hq, N, d = 2, 3, 10, 5
    q, kv = _rand((Sq, Hq, d), 71), _rand((N, d), 72)
    idx = np.array([[3, 7, 1, 9], [0, 2, 4, 8]], dtype=np.int32)
    base = orc.sparse_topk_attention(q, kv, idx, d_v=d, scale=0.4)
    perm = orc.sparse_topk_attention(q, kv, idx[:, ::-1].copy(), d_v=d, scale=0.4)
    worst = max(_err(base[0], perm[0]), _err(base[1], perm[1]))
    skip = orc.sparse_topk_attention(q, kv, np.array([[3, -1, 7, 1, 9, N], [0, 2, -5, 4, 8, 99]],
                                                     dtype=np.int32), d_v=d, scale=0.4)
    worst = max(worst, _err(base[0], skip[0]), _err(base[1], skip[1]))
    # duplicate index j: same as adding ln 2 to key j's score, done via an extra feature
    dup = orc.sparse_topk_attention(q, kv, np.array([[3, 7, 1, 9, 9], [0, 2, 4, 8, 8]], dtype=np.int32),
                                    d_v=d, scale=0.4)
    for s, j in ((0, 9), (1, 8)):
        sc = 0.4 * q[s] @ kv[idx[s]].T                   # [Hq, 4] scores, explicit
        sc[:, -1] += math.log(2.0)
        w = np.exp(sc - logsumexp(sc, axis=1, keepdims=True))
        worst = max(worst, _err(dup[0][s], w @ kv[idx[s]]), _err(dup[1][s], logsumexp(sc, axis=1)))
    # explicit gather equals a one-hot selection-matrix product
    sel = np.zeros((4, N))
    sel[np.arange(4), idx[0]] = 1.0
    worst = max(worst, _err(orc.gather_rows(kv, idx[0]), sel @ kv))
    return worst


def check_lse_logsumexp(orc=oracle):
    """lse equals log-sum-exp of the explicit scores (scipy), with exp(sink) included."""
    q, k, v = _rand((1, 3, 5, 4), 81), _rand((1, 1, 5, 4), 82), _rand((1, 1, 5, 2), 83)
    sinks = _rand((3,), 84)
    _, l = orc.dense_attention(q, k, v, scale=0.6, causal=False, sinks=sinks)
    worst = 0.0
    for h in range(3):
        s = 0.6 * q[0, h] @ k[0, 0].T
        ref = logsumexp(np.concatenate([s, np.full((5, 1), sinks[h])], axis=1), axis=1)
        worst = max(worst, _err(l[0, h], ref))
    return worst


def check_dropout(orc=oracle):
    """Dropout on the probabilities: brute force with the mask applied to the value
    rows (a different placement of the same factor), an all-kept mask with p = 0 is
    no dropout, an all-kept mask with p > 0 scales O by 1 / (1 - p), and lse never
    changes."""
    worst = 0.0
    rng = np.random.default_rng(990)
    for i, (B, H, Hkv, Tq, Tk, d) in enumerate([(1, 4, 2, 5, 7, 3), (2, 2, 1, 6, 4, 4)]):
        q, k, v = _rand((B, H, Tq, d), 991 + i, 0.8), _rand((B, Hkv, Tk, d), 992 + i, 0.8), _rand((B, Hkv, Tk, 2), 993 + i)
        sinks = _rand((H,), 994 + i)
        keep = rng.random((B, H, Tq, Tk)) > 0.3
        for causal in (False, True):
            for sk in (None, sinks):
                o, l = orc.dense_attention(q, k, v, scale=0.7, causal=causal, sinks=sk, keep=keep, p_drop=0.3)
                bo, bl = brute_dense(q, k, v, 0.7, causal, sk, keep=keep, p_drop=0.3)
                o0, l0 = orc.dense_attention(q, k, v, scale=0.7, causal=causal, sinks=sk)
                worst = max(worst, _err(o, bo), _err(l, bl), _err(l, l0))
                ones = np.ones_like(keep)
                o1, _ = orc.dense_attention(q, k, v, scale=0.7, causal=causal, sinks=sk, keep=ones, p_drop=0.0)
                o2, _ = orc.dense_attention(q, k, v, scale=0.7, causal=causal, sinks=sk, keep=ones, p_drop=0.25)
                worst = max(worst, _err(o1, o0), _err(o2, o0 / 0.75))
    return worst


def check_extras(orc=oracle):
    """The extra returns (probabilities, row maxima): brute force, P . V = O of the
    forward, and each row's probabilities plus the sink's share sum to 1."""
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, d) in enumerate([(1, 4, 2, 5, 7, 3), (2, 2, 1, 6, 4, 4)]):
        q, k = _rand((B, H, Tq, d), 970 + i, 0.8), _rand((B, Hkv, Tk, d), 971 + i, 0.8)
        v = _rand((B, Hkv, Tk, 2), 972 + i)
        sinks = _rand((H,), 973 + i)
        for causal in (False, True):
            for sk in (None, sinks):
                for win in ((-1, -1), (1, 0)):
                    P, M = orc.dense_attention_extras(q, k, scale=0.7, causal=causal, sinks=sk, window=win)
                    bP, bM = brute_extras(q, k, 0.7, causal, sk, window=win)
                    worst = max(worst, _err(P, bP), _err(M, bM))
                    o, l = orc.dense_attention(q, k, v, scale=0.7, causal=causal, sinks=sk, window=win)
                    worst = max(worst, _err(np.einsum("bhts,bhsd->bhtd", P, OA.repeat_kv(v, H // Hkv)), o))
                    share = 0.0 if sk is None else np.exp(sk[None, :, None] - l)
                    rows = P.sum(axis=-1) + np.where(np.isfinite(l), share, 0.0)
                    worst = max(worst, _err(np.where(np.isfinite(l), rows, 1.0), 1.0))
    return worst


def check_two_part(orc=oracle):
    """MLA's two-part rows: brute force that sums the two partial dot products in
    separate loops (no concatenation), with a rope key per kv head and one shared
    by all kv heads; and the shared case equals the concatenation with the rope
    key copied to every head."""
    worst = 0.0
    for i, (B, H, Hkv, Tq, Tk, dn, dr, dv) in enumerate([(1, 4, 2, 5, 7, 4, 3, 2), (2, 3, 3, 4, 4, 2, 2, 3)]):
        qn, qr = _rand((B, H, Tq, dn), 950 + i), _rand((B, H, Tq, dr), 951 + i)
        kn, v = _rand((B, Hkv, Tk, dn), 952 + i), _rand((B, Hkv, Tk, dv), 953 + i)
        sinks = _rand((H,), 954 + i)
        for kr in (_rand((B, Hkv, Tk, dr), 955 + i), _rand((B, 1, Tk, dr), 956 + i)):
            for causal in (False, True):
                for sk in (None, sinks):
                    o, l = orc.dense_attention_two_part(qn, qr, kn, kr, v, scale=0.6, causal=causal, sinks=sk)
                    bo, bl = brute_two_part(qn, qr, kn, kr, v, 0.6, causal, sk)
                    worst = max(worst, _err(o, bo), _err(l, bl))
    qn, qr = _rand((1, 4, 6, 3), 960), _rand((1, 4, 6, 2), 961)
    kn, kr, v = _rand((1, 2, 6, 3), 962), _rand((1, 1, 6, 2), 963), _rand((1, 2, 6, 2), 964)
    o, l = orc.dense_attention_two_part(qn, qr, kn, kr, v, scale=0.6, causal=True)
    kc = np.concatenate([kn, np.concatenate([kr, kr], axis=1)], axis=-1)
    o2, l2 = orc.dense_attention(np.concatenate([qn, qr], axis=-1), kc, v, scale=0.6, causal=True)
    return max(worst, _err(o, o2), _err(l, l2))


ALL_CHECKS = {
    "two_part": check_two_part,
    "extras": check_extras,
    "dropout": check_dropout,
    "window": check_window,
    "varlen": check_varlen,
    "brute_dense": check_brute_dense,
    "brute_sparse": check_brute_sparse,
    "library_dense": check_library_dense,
    "closed_forms": check_closed_forms,
    "causal_differs": check_causal_differs,
    "fully_masked_rows": check_fully_masked_rows,
    "fold_matches_repeat_kv": check_fold_matches_repeat_kv,
    "tiling_exact": check_tiling_exact,
    "sink_limit": check_sink_limit,
    "shift_invariance": check_shift_invariance,
    "kv_split_merge": check_kv_split_merge,
    "sparse_equals_dense_mqa": check_sparse_equals_dense_mqa,
    "sparse_conventions": check_sparse_conventions,
    "lse_logsumexp": check_lse_logsumexp,
}
