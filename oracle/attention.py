"""fp64 CPU oracle for the fused attention forward and its backward.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the bench's
CPU-baseline leg may import this module. It shares no code with the HIP path:
it is the plain definition written out, slow and explicit, so that a reader can
check it against the pages by eye.

What it computes, and the passage each part follows:

* The attention forward returns the output together with the per-row
  log-sum-exp (pith-train page, "Issues resolved" item 1: FA4's forward returns
  ``(out, lse)``).
* GQA/MQA: the K/V heads are expanded by ``repeat_kv`` with kv-major heads,
  ``y[b, kv*n_rep + rep] = x[b, kv]`` (ArcFlash page, "What rung 0 does"). The
  oracle performs that expansion as an explicit copy.
* Sinks: a per-head constant that enters each row's softmax denominator and
  nothing else (ArcFlash page, "What rung 0 does", last paragraph; the "sink
  dropped from the softmax denominator" mutation under "Mutations").
* Query-row tiling under a byte budget is exact because each output row is an
  independent softmax (ArcFlash page, "What rung 0 does").
* MLA asymmetric head dims: q and k carry d_qk, v carries d_v (pith-train page,
  "Issues resolved" item 2: the no-rope/rope concatenation is done by the
  caller and fed to the attention directly).
* Sparse top-k: each query attends only to the rows of one shared KV pool that
  its index list names (TensorRT-LLM page, "Description": 13312 queries x 64
  heads x 2176 top-k rows, d_qk 512).
* Backward: the Q/K/V gradients that a raw attention backward returns after
  the forward and the output merge (TransformerEngine page, "Flowchart" and
  "Summary": raw forward/backward wrappers with LSE handling). The pages give
  no formulas; the oracle is the chain rule through the forward definition
  above, written out step by step (and the sink's gradient, since the sink is
  a per-head parameter of the same softmax).

Readings where the pages are silent (each one stated again where it is used):

* The sink is a logit in the scaled-score space: it is not multiplied by
  ``scale``.
* ``lse`` is the natural log of the full denominator, so it includes the sink
  term when sinks are given.
* Causal masks are bottom-right aligned: key j is visible to query t iff
  ``j <= t + (Tk - Tq)``.
* A row with no visible key has O = 0 and lse = -inf (lse = sink with a sink).
* Sparse: ``V = kv[:, :d_v]`` of the one pool (V == K when d_v == d_qk); an
  index outside [0, N) is skipped; duplicates count with multiplicity.

Every function here is pinned by tests against brute force, closed forms,
library routines and invariants. Two conventions are readings that the pages
do not fix at all: the sink term inside lse, and the skipped out-of-range
sparse index. Their closed-form tests pin the code to the stated reading, not
to the pages, so those two conventions are "parity unpinned" as far as the
pages go; the configurations exercise neither of them except the sink in lse.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Exact upcast to fp64 (bf16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def repeat_kv(x: np.ndarray, n_rep: int) -> np.ndarray:
    """Explicit GQA expansion with kv-major heads: ``y[b, kv*n_rep + rep] = x[b, kv]``.

    ArcFlash page, "What rung 0 does" (the repeat_kv mapping). This is the copy
    that the fused path avoids; the oracle performs it on purpose.
    """
    B, Hkv, T, D = x.shape
    y = np.empty((B, Hkv * n_rep, T, D), dtype=x.dtype)
    for kv in range(Hkv):
        for rep in range(n_rep):
            y[:, kv * n_rep + rep] = x[:, kv]
    return y


def _causal_mask(ts, Tq: int, Tk: int) -> np.ndarray:
    """Boolean [len(ts), Tk]: True where key j is visible to query token t."""
    j = np.arange(Tk)[None, :]
    t = np.asarray(ts)[:, None]
    return j <= t + (Tk - Tq)


def _window_mask(ts, Tq: int, Tk: int, left: int, right: int) -> np.ndarray:
    """Boolean [len(ts), Tk]: True where key j lies in the sliding window of token t.

    The window is centred on the bottom-right diagonal position t + (Tk - Tq):
    ``left`` keys before it and ``right`` keys after it, a negative value
    meaning unbounded on that side (the (left, right) window arguments that
    TransformerEngine's FA4 path forwards, TE page "Summary").
    """
    j = np.arange(Tk)[None, :]
    c = np.asarray(ts)[:, None] + (Tk - Tq)
    keep = np.ones((len(ts), Tk), dtype=bool)
    if left >= 0:
        keep &= j >= c - left
    if right >= 0:
        keep &= j <= c + right
    return keep


def _tile_row_token(f: np.ndarray, f0: int, Tq: int) -> np.ndarray:
    """Token index of folded rows ``f`` (a tile starting at folded row ``f0``).

    The token depends on the folded row alone, never on where the tile starts:
    "the mask follows the tile" (ArcFlash page, "Mutations").
    """
    return f % Tq


def _value_rows(G: np.ndarray, d_v: int) -> np.ndarray:
    """V rows of gathered pool rows: the first d_v columns (V == K when d_v == d_qk)."""
    return G[:, :d_v]


def _softmax_rows(S: np.ndarray, sink: Optional[float]) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of an explicit score matrix ``S`` [R, n] (masked entries = -inf).

    Returns the probabilities P [R, n] and lse [R]. With a sink s, the row
    denominator gains exp(s) and nothing else does (ArcFlash page, sinks).
    """
    R = S.shape[0]
    m = S.max(axis=1) if S.shape[1] > 0 else np.full(R, NEG_INF)
    if sink is not None:
        m = np.maximum(m, sink)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    E = np.exp(S - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    denom = E.sum(axis=1)
    if sink is not None:
        denom = denom + np.exp(sink - m_safe)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(denom[:, None] > 0, E / np.where(denom > 0, denom, 1.0)[:, None], 0.0)
        lse = np.where(denom > 0, m_safe + np.log(np.where(denom > 0, denom, 1.0)), NEG_INF)
    return P, lse


def dense_attention(q, k, v, *, scale: float, causal: bool, sinks=None,
                    rows: Optional[Iterable[Tuple[int, int, int]]] = None, window: Tuple[int, int] = (-1, -1),
                    keep=None, p_drop: float = 0.0):
    """Dense attention forward in fp64.

    q [B,H,Tq,d_qk], k [B,Hkv,Tk,d_qk], v [B,Hkv,Tk,d_v], sinks [H] or None.
    Returns (out [B,H,Tq,d_v], lse [B,H,Tq]) -- or, when ``rows`` lists
    (b, h, t) triples, (out [n, d_v], lse [n]) for those rows only.

    Steps (explicit, in the order of the definition):
      1. K, V expanded to H heads by repeat_kv (kv-major).
      2. S = scale * q . K^T, an explicit [Tq, Tk] score matrix per (b, h).
      3. Causal: S[t, j] = -inf where j > t + (Tk - Tq). Sliding window
         (left, right): also -inf outside [c - left, c + right] with
         c = t + (Tk - Tq); a negative bound is no bound. The window never
         widens the causal mask (the ArcFlash page, "What this does NOT do",
         names a window clamp that turned causal attention into full
         attention as a defect).
      4. Row softmax with the sink (if any) added to the denominator only.
      5. O = P . V;  lse = m + ln(denominator).
    Dropout (``keep`` [B,H,Tq,Tk] bool, probability ``p_drop``): the
    probabilities are multiplied by keep / (1 - p_drop) before the product
    with V; lse stays that of the softmax (the dropout acts after it).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, Dqk = q.shape
    _, Hkv, Tk, _ = k.shape
    Dv = v.shape[-1]
    assert H % Hkv == 0, "H must be a multiple of Hkv"
    g = H // Hkv
    K = repeat_kv(k, g)
    V = repeat_kv(v, g)
    sk = None if sinks is None else _f64(sinks)
    keep = None if keep is None else np.asarray(keep, dtype=bool)

    def head(b, h, ts):
        S = scale * (q[b, h, ts] @ K[b, h].T)
        if causal:
            S = np.where(_causal_mask(ts, Tq, Tk), S, NEG_INF)
        if window[0] >= 0 or window[1] >= 0:
            S = np.where(_window_mask(ts, Tq, Tk, window[0], window[1]), S, NEG_INF)
        P, lse = _softmax_rows(S, None if sk is None else float(sk[h]))
        if keep is not None:
            P = _dropout(P, keep[b, h][ts], p_drop)
        return P @ V[b, h], lse

    if rows is None:
        out = np.empty((B, H, Tq, Dv))
        lse = np.empty((B, H, Tq))
        all_t = np.arange(Tq)
        for b in range(B):
            for h in range(H):
                out[b, h], lse[b, h] = head(b, h, all_t)
        return out, lse

    rows = list(rows)
    out = np.empty((len(rows), Dv))
    lse = np.empty(len(rows))
    # group the requested rows by (b, h) so each head's scores are formed once
    by_head = {}
    for i, (b, h, t) in enumerate(rows):
        by_head.setdefault((b, h), []).append((i, t))
    for (b, h), lst in by_head.items():
        ts = np.array([t for _, t in lst])
        o, l = head(b, h, ts)
        for r, (i, _) in enumerate(lst):
            out[i], lse[i] = o[r], l[r]
    return out, lse


def dense_attention_extras(q, k, *, scale: float, causal: bool, sinks=None, window: Tuple[int, int] = (-1, -1)):
    """The two extra returns FA4 b19 added to its forward (pith-train page, "Issues
    resolved" item 1: (out, lse) widened to (out, lse, p, row_max)), read as:

      p       [B,H,Tq,Tk]  the softmax probabilities exp(S - lse) of the visible
                           keys (0 where masked); the sink has no column, so with
                           sinks a row sums to 1 - exp(sink - lse)
      row_max [B,H,Tq]     the largest visible scaled score max_j S[t, j] (the
                           sink is not a score; -inf for a row with no key)

    with S = scale * q . K^T (repeat_kv, masks and lse as in ``dense_attention``).
    """
    q, k = _f64(q), _f64(k)
    B, H, Tq, _ = q.shape
    _, Hkv, Tk, _ = k.shape
    g = H // Hkv
    K = repeat_kv(k, g)
    sk = None if sinks is None else _f64(sinks)
    P = np.zeros((B, H, Tq, Tk))
    row_max = np.full((B, H, Tq), NEG_INF)
    ts = np.arange(Tq)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ K[b, h].T)
            if causal:
                S = np.where(_causal_mask(ts, Tq, Tk), S, NEG_INF)
            if window[0] >= 0 or window[1] >= 0:
                S = np.where(_window_mask(ts, Tq, Tk, window[0], window[1]), S, NEG_INF)
            P[b, h], _ = _softmax_rows(S, None if sk is None else float(sk[h]))
            if Tk > 0:
                row_max[b, h] = S.max(axis=1)
    return P, row_max


def dense_attention_two_part(q_nope, q_rope, k_nope, k_rope, v, *, scale: float, causal: bool, sinks=None,
                             window: Tuple[int, int] = (-1, -1)):
    """MLA's two-part rows (pith-train page, "Issues resolved" item 2: the model
    concatenates the no-rope and rope parts and feeds the result to the
    attention): the query row is [q_nope || q_rope] and the key row
    [k_nope || k_rope]. k_rope is [B, Hkv, Tk, r], or [B, 1, Tk, r] for one rope
    key shared by every kv head (MLA's decoupled rope key), which is copied to
    each kv head first. Then the dense definition on the concatenated rows.
    """
    q_nope, q_rope, k_nope, k_rope = _f64(q_nope), _f64(q_rope), _f64(k_nope), _f64(k_rope)
    Hkv = k_nope.shape[1]
    if k_rope.shape[1] == 1 and Hkv > 1:
        k_rope = np.repeat(k_rope, Hkv, axis=1)
    q = np.concatenate([q_nope, q_rope], axis=-1)
    k = np.concatenate([k_nope, k_rope], axis=-1)
    return dense_attention(q, k, v, scale=scale, causal=causal, sinks=sinks, window=window)


def dense_attention_varlen(q, k, v, cu_q, cu_k, *, scale: float, causal: bool, sinks=None,
                           window: Tuple[int, int] = (-1, -1)):
    """Packed variable-length batch: sequence b owns query tokens
    [cu_q[b], cu_q[b+1]) of q [total_q, H, d_qk] and key tokens
    [cu_k[b], cu_k[b+1]) of k, v [total_k, Hkv, d]. Each sequence is an
    independent dense attention (its own bottom-right causal alignment,
    window and sinks); no token attends across a sequence boundary. The
    ArcFlash page ("What this does NOT do") lists a varlen path that silently
    dropped the causal mask as a defect; here the mask applies per sequence.
    Returns (out [total_q, H, d_v], lse [H, total_q]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q = [int(x) for x in np.asarray(cu_q)]
    cu_k = [int(x) for x in np.asarray(cu_k)]
    total_q, H, _ = q.shape
    Dv = v.shape[-1]
    out = np.zeros((total_q, H, Dv))
    lse = np.full((H, total_q), NEG_INF)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe <= qs:
            continue
        qb = q[qs:qe].transpose(1, 0, 2)[None]            # [1, H, Tq_b, d]
        kb = k[ks:ke].transpose(1, 0, 2)[None]
        vb = v[ks:ke].transpose(1, 0, 2)[None]
        o, l = dense_attention(qb, kb, vb, scale=scale, causal=causal, sinks=sinks, window=window)
        out[qs:qe] = o[0].transpose(1, 0, 2)
        lse[:, qs:qe] = l[0]
    return out, lse


def tile_rows_for_budget(tile_bytes: int, Tk: int, elt_bytes: int) -> int:
    """Folded query rows per tile so that one tile's [rows, Tk] scores fit the budget.

    ArcFlash page, "What rung 0 does": the score matrix is bounded to one
    query tile of ``tile_bytes`` (32 MiB by default).
    """
    return max(1, tile_bytes // (Tk * elt_bytes))


def dense_attention_tiled(q, k, v, *, scale: float, causal: bool, sinks=None,
                          tile_bytes: int = 32 << 20):
    """The same forward computed over query-row tiles of the folded view.

    GQA fold: q [B,H,Tq,D] is viewed as [B,Hkv,g*Tq,D] (kv-major heads, so a
    contiguous reshape, ArcFlash page "What rung 0 does"); folded row f of kv
    head ``kv`` is head ``kv*g + f // Tq`` at token ``t = f % Tq``. Tiles of
    ``tile_rows`` folded rows may straddle heads; each row's causal bound uses
    its own ``t`` ("the mask follows the tile") and its own head's sink.
    K and V are used per kv head, without expansion. fp64 scores are 8 bytes.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, Dqk = q.shape
    _, Hkv, Tk, _ = k.shape
    Dv = v.shape[-1]
    g = H // Hkv
    qf = q.reshape(B, Hkv, g * Tq, Dqk)       # the fold: a view, no copy
    sk = None if sinks is None else _f64(sinks)
    rows_per_tile = tile_rows_for_budget(tile_bytes, Tk, 8)
    out = np.empty((B, Hkv, g * Tq, Dv))
    lse = np.empty((B, Hkv, g * Tq))
    for b in range(B):
        for kv in range(Hkv):
            for f0 in range(0, g * Tq, rows_per_tile):
                f = np.arange(f0, min(f0 + rows_per_tile, g * Tq))
                t = _tile_row_token(f, f0, Tq)
                h = kv * g + f // Tq
                S = scale * (qf[b, kv, f] @ k[b, kv].T)
                if causal:
                    S = np.where(_causal_mask(t, Tq, Tk), S, NEG_INF)
                # rows of one tile can belong to different heads: softmax per head
                P = np.empty_like(S)
                L = np.empty(len(f))
                for hh in np.unique(h):
                    sel = h == hh
                    P[sel], L[sel] = _softmax_rows(S[sel], None if sk is None else float(sk[hh]))
                out[b, kv, f] = P @ v[b, kv]
                lse[b, kv, f] = L
    return out.reshape(B, H, Tq, Dv), lse.reshape(B, H, Tq)


def gather_rows(pool: np.ndarray, idx: Sequence[int]) -> np.ndarray:
    """Explicit gather ``pool[idx]`` that skips indices outside [0, N)."""
    N = pool.shape[0]
    keep = [int(i) for i in idx if 0 <= int(i) < N]
    return pool[np.asarray(keep, dtype=np.int64)] if keep else pool[:0]


def sparse_topk_attention(q, kv, idx, *, d_v: int, scale: float, sinks=None,
                          queries: Optional[Iterable[int]] = None):
    """Sparse top-k forward in fp64.

    q [Sq,Hq,d_qk], kv [N,d_qk] (one shared pool), idx [Sq,topk] integer.
    V is the first d_v columns of the same pool (V == K when d_v == d_qk).
    For query s: G = kv[idx[s]] (explicit gather), S = scale * q[s] . G^T
    ([Hq, topk], no mask), row softmax (sink in the denominator only),
    O = P . G[:, :d_v]. Returns (out [Sq,Hq,d_v], lse [Sq,Hq]) or, with
    ``queries``, (out [n,Hq,d_v], lse [n,Hq]) for those queries.
    """
    q, kv = _f64(q), _f64(kv)
    idx = np.asarray(idx.numpy() if hasattr(idx, "numpy") else idx)
    Sq, Hq, Dqk = q.shape
    sk = None if sinks is None else _f64(sinks)
    qs = list(range(Sq)) if queries is None else list(queries)
    out = np.empty((len(qs), Hq, d_v))
    lse = np.empty((len(qs), Hq))
    for i, s in enumerate(qs):
        G = gather_rows(kv, idx[s])
        S = scale * (q[s] @ G.T)                      # [Hq, n]
        Vg = _value_rows(G, d_v)
        for h in range(Hq):
            P, L = _softmax_rows(S[h:h + 1], None if sk is None else float(sk[h]))
            out[i, h] = P[0] @ Vg
            lse[i, h] = L[0]
    return out, lse


def dequantize_rows(raw, fmt: str) -> np.ndarray:
    """Decode a quantized cache [..., row bytes] (uint8) into fp64 values [..., d].

    The cache types the llama.cpp page names (q8_0 / q4_0 K/V, "Pins #303") are
    ggml's block formats; the pages name them without spelling them out, so
    this follows their public definition: blocks of 32 values, each an fp16
    scale d then the codes. q8_0 (34 bytes): value i = d * int8 code i.
    q4_0 (18 bytes): code i is the low nibble of byte i for i < 16 and the high
    nibble of byte i - 16 otherwise, value = d * (code - 8).
    """
    a = np.asarray(raw.numpy() if hasattr(raw, "numpy") else raw, dtype=np.uint8)
    bb = {"q8_0": 34, "q4_0": 18}[fmt]
    lead, rb = a.shape[:-1], a.shape[-1]
    assert rb % bb == 0
    nb = rb // bb
    blocks = a.reshape(-1, nb, bb)
    d = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)  # [n, nb]
    if fmt == "q8_0":
        codes = blocks[..., 2:].view(np.int8).astype(np.float64)           # [n, nb, 32]
    else:
        bytes_ = blocks[..., 2:].astype(np.int64)                           # [n, nb, 16]
        lo, hi = bytes_ & 0xF, bytes_ >> 4
        codes = np.concatenate([lo, hi], axis=-1).astype(np.float64) - 8.0  # elements 0..15, 16..31
    vals = d[..., None] * codes
    return vals.reshape(*lead, nb * 32)


def decode_fp8_e4m3(codes) -> np.ndarray:
    """OCP FP8 E4M3 bytes -> fp64, from the format's definition: sign bit 7, exponent
    bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is subnormal (m / 8 * 2^-6);
    the pattern S.1111.111 is NaN; there are no infinities (largest finite 448)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def dequantize_fp8_rows(codes, scales, block: int = 128) -> np.ndarray:
    """Pool rows stored as fp8 codes [N, d] with one scale per ``block`` columns
    [N, d / block]: value = decode(code) * scale of its block."""
    v = decode_fp8_e4m3(codes)
    sc = np.repeat(_f64(scales), block, axis=1)
    return v * sc


def merge_partials(parts, sink: Optional[float] = None):
    """Merge (O_i, lse_i) computed over disjoint key sets into the full result.

    lse = log(sum_i exp(lse_i) [+ exp(sink)]), O = sum_i exp(lse_i - lse) O_i.
    Each part must have been computed without the sink. This is the output
    merge of context-parallel attention (TransformerEngine page, flowchart:
    "ring communication and output merge"), done on one device.
    """
    lses = np.stack([p[1] for p in parts])            # [n, R]
    terms = list(lses)
    if sink is not None:
        terms.append(np.full_like(lses[0], sink))
    allt = np.stack(terms)
    m = allt.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    tot = np.exp(allt - m_safe).sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    out = np.zeros_like(parts[0][0])
    for o, l in parts:
        w = np.where(np.isfinite(l), np.exp(l - lse_safe), 0.0)
        out = out + w[..., None] * o
    return out, lse


def _dropout(P: np.ndarray, keep: np.ndarray, p_drop: float) -> np.ndarray:
    """Attention dropout on the probabilities: kept entries scaled by 1 / (1 - p), the
    others zeroed (the TransformerEngine page's review names dropout_p and the RNG
    state that the forward and the backward must share; here the mask itself is the
    shared input)."""
    return np.where(keep, P / (1.0 - p_drop), 0.0)


def _softmax_backward(P: np.ndarray, dP: np.ndarray, dO: np.ndarray, O: np.ndarray) -> np.ndarray:
    """dS = P * (dP - D) with D = rowsum(dO * O): the softmax Jacobian applied to dP.

    With a sink the rows of P sum to 1 - p_sink; the Jacobian of the visible
    entries is still P * (dP - sum_j P_j dP_j), and sum_j P_j dP_j = rowsum(dO * O)
    because O = P . V.
    """
    D = (dO * O).sum(axis=1)
    return P * (dP - D[:, None])


def sum_kv_groups(x: np.ndarray, g: int) -> np.ndarray:
    """Adjoint of ``repeat_kv``: ``y[b, kv] = sum_rep x[b, kv*g + rep]`` (kv-major heads)."""
    B, H, T, D = x.shape
    y = np.zeros((B, H // g, T, D), dtype=x.dtype)
    for kv in range(H // g):
        for rep in range(g):
            y[:, kv] += x[:, kv * g + rep]
    return y


def dense_attention_backward(q, k, v, dout, *, scale: float, causal: bool, sinks=None,
                             window: Tuple[int, int] = (-1, -1), keep=None, p_drop: float = 0.0):
    """Gradients of the dense forward in fp64: (dq, dk, dv, dsinks).

    ``dout`` = dL/dO [B,H,Tq,d_v] for a scalar loss L of the output; the lse
    output is a saved statistic and carries no gradient. dsinks is None when
    ``sinks`` is None. Steps, per (b, h), through the forward's definition:

      1. Recompute the forward: S = scale * q . K_h^T (explicit, masked by the
         causal bound and the sliding window as in the forward), the row
         softmax P with the sink in the denominator, O = P . V_h.
      2. dV_h = P^T . dO                      (O is linear in V)
      3. dP = dO . V_h^T                      (O is linear in P)
      4. D = rowsum(dO * O)                   (= rowsum(P * dP))
      5. dS = P * (dP - D)                    (softmax Jacobian, sink included:
                                               the sink only enlarges the
                                               denominator, so it appears in P
                                               and D but has no column)
      6. dq = scale * dS . K_h,  dK_h = scale * dS^T . q
      7. dsink_h = -sum over rows of p_sink * D, with p_sink = exp(sink - lse)
      8. dk, dv of kv head kv = sum of dK_h, dV_h over the g heads that read
         it (the adjoint of repeat_kv's kv-major copy).
    With dropout (``keep``, ``p_drop`` as in the forward) the product with V
    takes Pd = P * keep / (1 - p): dV = Pd^T dO, O = Pd V, and the chain rule
    through the mask gives dS = P * (dPd - D) with dPd = (dO V^T) * keep / (1 - p)
    (D = rowsum(dO * O) of the dropped output, as before).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Tq, Dqk = q.shape
    _, Hkv, Tk, _ = k.shape
    Dv = v.shape[-1]
    assert H % Hkv == 0, "H must be a multiple of Hkv"
    g = H // Hkv
    K = repeat_kv(k, g)
    V = repeat_kv(v, g)
    sk = None if sinks is None else _f64(sinks)
    dq = np.zeros_like(q)
    dK = np.zeros((B, H, Tk, Dqk))
    dV = np.zeros((B, H, Tk, Dv))
    dsk = None if sk is None else np.zeros(H)
    ts = np.arange(Tq)
    keep = None if keep is None else np.asarray(keep, dtype=bool)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ K[b, h].T)
            if causal:
                S = np.where(_causal_mask(ts, Tq, Tk), S, NEG_INF)
            if window[0] >= 0 or window[1] >= 0:
                S = np.where(_window_mask(ts, Tq, Tk, window[0], window[1]), S, NEG_INF)
            sink = None if sk is None else float(sk[h])
            P, lse = _softmax_rows(S, sink)
            Pd = P if keep is None else _dropout(P, keep[b, h], p_drop)
            O = Pd @ V[b, h]
            dO = dout[b, h]
            dV[b, h] = Pd.T @ dO
            dP = dO @ V[b, h].T
            if keep is not None:
                dP = _dropout(dP, keep[b, h], p_drop)
            dS = _softmax_backward(P, dP, dO, O)
            dq[b, h] = scale * (dS @ K[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h])
            if sink is not None:
                D = (dO * O).sum(axis=1)
                p_sink = np.where(np.isfinite(lse), np.exp(sink - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
                dsk[h] -= float((p_sink * D).sum())
    return dq, sum_kv_groups(dK, g), sum_kv_groups(dV, g), dsk


def scatter_add_rows(y: np.ndarray, idx: Sequence[int], rows: np.ndarray) -> None:
    """Adjoint of ``gather_rows``, accumulated into ``y``: y[n] += rows[j] for every slot j
    with idx[j] == n, in slot order (slots whose index is outside [0, len(y)) contribute
    nothing, as they were skipped)."""
    for j, n in enumerate(idx):
        n = int(n)
        if 0 <= n < y.shape[0]:
            y[n] += rows[j]


def sparse_topk_attention_backward(q, kv, idx, dout, *, d_v: int, scale: float, sinks=None):
    """Gradients of the sparse top-k forward in fp64: (dq, dkv, dsinks).

    ``dout`` = dL/dO [Sq,Hq,d_v]; lse carries no gradient (as in the dense
    backward). The pool plays both roles: its rows are the keys (all d_qk
    columns) and their first d_v columns the values, so the pool's gradient is
    the sum of the two. Per query s, through the forward's definition:

      1. G = kv[idx[s]] (explicit gather, skipped slots dropped),
         S = scale * q[s] . G^T, row softmax P (sink in the denominator),
         O = P . G[:, :d_v].
      2. dP = dO . G[:, :d_v]^T, D = rowsum(dO * O), dS = P * (dP - D).
      3. dq[s] = scale * dS . G.
      4. dG = scale * dS^T . q[s]            (key role, all d_qk columns)
         dG[:, :d_v] += P^T . dO             (value role)
      5. dkv += the scatter-add of dG into the rows idx[s] names (the adjoint
         of the gather; a duplicated index receives both slots' gradients).
      6. dsink_h = -sum over queries of exp(sink_h - lse) * D.
    """
    q, kv, dout = _f64(q), _f64(kv), _f64(dout)
    idx = np.asarray(idx.numpy() if hasattr(idx, "numpy") else idx)
    Sq, Hq, Dqk = q.shape
    N = kv.shape[0]
    sk = None if sinks is None else _f64(sinks)
    dq = np.zeros_like(q)
    dkv = np.zeros((N, Dqk))
    dsk = None if sk is None else np.zeros(Hq)
    for s in range(Sq):
        keep = [int(n) for n in idx[s] if 0 <= int(n) < N]
        G = gather_rows(kv, keep)
        Vg = _value_rows(G, d_v)
        S = scale * (q[s] @ G.T)                                  # [Hq, n]
        P = np.empty_like(S)
        lse = np.empty(Hq)
        for h in range(Hq):
            Ph, Lh = _softmax_rows(S[h:h + 1], None if sk is None else float(sk[h]))
            P[h], lse[h] = Ph[0], Lh[0]
        O = P @ Vg
        dO = dout[s]
        dP = dO @ Vg.T
        dS = _softmax_backward(P, dP, dO, O)
        dq[s] = scale * (dS @ G)
        dG = scale * (dS.T @ q[s])
        dG[:, :d_v] += P.T @ dO
        scatter_add_rows(dkv, keep, dG)
        if sk is not None:
            D = (dO * O).sum(axis=1)
            fin = np.isfinite(lse)
            p_sink = np.where(fin, np.exp(sk - np.where(fin, lse, 0.0)), 0.0)
            dsk -= p_sink * D
    return dq, dkv, dsk
