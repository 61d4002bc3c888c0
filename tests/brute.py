"""Brute-force attention in pure Python, for pinning the oracle on tiny inputs.

Written independently of ``oracle/``: scores by explicit loops with
``math.fsum``, the GQA head mapping as ``kv = h // g`` (no expansion), and the
softmax in a different algebraic form -- the weight of key j is
``1 / (sum_i exp(s_i - s_j) + exp(sink - s_j))`` -- with lse taken unshifted as
``log(fsum(exp(s_i)) + exp(sink))`` (inputs are kept small so nothing
overflows). Mask: key j visible to token t iff j <= t + (Tk - Tq).
"""
import math


def _attend(scores, values, sink):
    """scores: list of floats; values: list of rows. Returns (o, lse)."""
    dv = len(values[0]) if values else 0
    if not scores:
        return None, (sink if sink is not None else -math.inf)
    w = []
    for sj in scores:
        terms = [math.exp(si - sj) for si in scores]
        if sink is not None:
            terms.append(math.exp(sink - sj))
        w.append(1.0 / math.fsum(terms))
    o = [math.fsum(w[j] * values[j][d] for j in range(len(scores))) for d in range(dv)]
    tot = [math.exp(si) for si in scores]
    if sink is not None:
        tot.append(math.exp(sink))
    return o, math.log(math.fsum(tot))


def brute_dense(q, k, v, scale, causal, sinks=None, window=(-1, -1), keep=None, p_drop=0.0):
    """q [B][H][Tq][Dqk], k [B][Hkv][Tk][Dqk], v [B][Hkv][Tk][Dv] (nested lists or arrays).
    window (left, right): key j kept iff left < 0 or j >= t + Tk - Tq - left, and
    right < 0 or j <= t + Tk - Tq + right (tested key by key)."""
    B, H, Tq, Dqk = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Tk, Dv = len(k[0]), len(k[0][0]), len(v[0][0][0])
    g = H // Hkv
    out = [[[[0.0] * Dv for _ in range(Tq)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * Tq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            kvh = h // g
            for t in range(Tq):
                sc, vals = [], []
                for j in range(Tk):
                    if causal and j > t + (Tk - Tq):
                        continue
                    if window[0] >= 0 and t + (Tk - Tq) - j > window[0]:
                        continue
                    if window[1] >= 0 and j - (t + (Tk - Tq)) > window[1]:
                        continue
                    sc.append(scale * math.fsum(float(q[b][h][t][d]) * float(k[b][kvh][j][d])
                                                for d in range(Dqk)))
                    # dropout: a dropped key's value row is zero, a kept one is scaled
                    z = 1.0 if keep is None else (1.0 / (1.0 - p_drop) if keep[b][h][t][j] else 0.0)
                    vals.append([z * float(x) for x in v[b][kvh][j]])
                o, l = _attend(sc, vals, None if sinks is None else float(sinks[h]))
                out[b][h][t] = o if o is not None else [0.0] * Dv
                lse[b][h][t] = l
    return out, lse


def brute_sparse(q, kv, idx, d_v, scale, sinks=None):
    """q [Sq][Hq][Dqk], kv [N][Dqk], idx [Sq][topk]; out-of-range indices skipped."""
    Sq, Hq, Dqk = len(q), len(q[0]), len(q[0][0])
    N = len(kv)
    out = [[[0.0] * d_v for _ in range(Hq)] for _ in range(Sq)]
    lse = [[0.0] * Hq for _ in range(Sq)]
    for s in range(Sq):
        rows = [int(i) for i in idx[s] if 0 <= int(i) < N]
        for h in range(Hq):
            sc = [scale * math.fsum(float(q[s][h][d]) * float(kv[r][d]) for d in range(Dqk))
                  for r in rows]
            vals = [[float(kv[r][d]) for d in range(d_v)] for r in rows]
            o, l = _attend(sc, vals, None if sinks is None else float(sinks[h]))
            out[s][h] = o if o is not None else [0.0] * d_v
            lse[s][h] = l
    return out, lse


def brute_two_part(qn, qr, kn, kr, v, scale, causal, sinks=None):
    """Two-part rows without concatenation: score = scale * (sum over the no-rope
    columns + sum over the rope columns), each part by its own loop; the rope key
    of kv head kvh is kr[b][kvh], or kr[b][0] when kr has one head (shared)."""
    B, H, Tq = len(qn), len(qn[0]), len(qn[0][0])
    Hkv, Tk, Dv = len(kn[0]), len(kn[0][0]), len(v[0][0][0])
    g = H // Hkv
    out = [[[None] * Tq for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * Tq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            kvh = h // g
            rh = 0 if len(kr[b]) == 1 else kvh
            for t in range(Tq):
                sc, vals = [], []
                for j in range(Tk):
                    if causal and j > t + (Tk - Tq):
                        continue
                    a = math.fsum(float(x) * float(y) for x, y in zip(qn[b][h][t], kn[b][kvh][j]))
                    r = math.fsum(float(x) * float(y) for x, y in zip(qr[b][h][t], kr[b][rh][j]))
                    sc.append(scale * (a + r))
                    vals.append([float(x) for x in v[b][kvh][j]])
                o, l = _attend(sc, vals, None if sinks is None else float(sinks[h]))
                out[b][h][t] = o if o is not None else [0.0] * Dv
                lse[b][h][t] = l
    return out, lse


def brute_extras(q, k, scale, causal, sinks=None, window=(-1, -1)):
    """Probabilities and row maxima by explicit loops: for each row, the visible
    keys' scores by fsum, weight of key j = 1 / (sum_i exp(s_i - s_j) + exp(sink - s_j))
    (0 for masked keys), row max = the largest visible score (-inf if none)."""
    B, H, Tq = len(q), len(q[0]), len(q[0][0])
    Hkv, Tk = len(k[0]), len(k[0][0])
    g = H // Hkv
    P = [[[[0.0] * Tk for _ in range(Tq)] for _ in range(H)] for _ in range(B)]
    M = [[[-math.inf] * Tq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            kvh = h // g
            for t in range(Tq):
                keys, sc = [], []
                for j in range(Tk):
                    if causal and j > t + (Tk - Tq):
                        continue
                    if window[0] >= 0 and t + (Tk - Tq) - j > window[0]:
                        continue
                    if window[1] >= 0 and j - (t + (Tk - Tq)) > window[1]:
                        continue
                    keys.append(j)
                    sc.append(scale * math.fsum(float(x) * float(y) for x, y in zip(q[b][h][t], k[b][kvh][j])))
                for j, sj in zip(keys, sc):
                    terms = [math.exp(si - sj) for si in sc]
                    if sinks is not None:
                        terms.append(math.exp(float(sinks[h]) - sj))
                    P[b][h][t][j] = 1.0 / math.fsum(terms)
                if sc:
                    M[b][h][t] = max(sc)
    return P, M
