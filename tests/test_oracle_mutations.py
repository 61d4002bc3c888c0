"""Planted mistakes in the oracle must each be caught by some pin.

The four mutations of the ArcFlash page ("Mutations": rep-major heads, mask not
following the tile, sink dropped from the denominator, and a disabled fast path
-- the last one is covered by the dispatch-record tests of the library) plus
causal switched off, scale applied twice, lse in base 2 and V taken from the
wrong columns of the sparse pool. Mistakes are planted on the CPU only.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as OA
from tests import pins


def _caught(checks):
    return {n: pins.ALL_CHECKS[n]() for n in checks}


def _assert_caught(results):
    assert any(v > pins.TOL for v in results.values()), f"mutation not caught: {results}"


def test_rep_major_heads_caught(monkeypatch):
    def rep_major(x, n_rep):
        B, Hkv, T, D = x.shape
        y = np.empty((B, Hkv * n_rep, T, D), dtype=x.dtype)
        for kv in range(Hkv):
            for rep in range(n_rep):
                y[:, rep * Hkv + kv] = x[:, kv]
        return y

    monkeypatch.setattr(OA, "repeat_kv", rep_major)
    _assert_caught(_caught(["fold_matches_repeat_kv", "brute_dense"]))


def test_mask_not_following_tile_caught(monkeypatch):
    monkeypatch.setattr(OA, "_tile_row_token", lambda f, f0, Tq: (f - f0) % Tq)
    _assert_caught(_caught(["tiling_exact"]))


def test_sink_dropped_caught(monkeypatch):
    orig = OA._softmax_rows
    monkeypatch.setattr(OA, "_softmax_rows", lambda S, sink: orig(S, None))
    _assert_caught(_caught(["closed_forms", "brute_dense", "lse_logsumexp"]))


def test_causal_off_caught(monkeypatch):
    monkeypatch.setattr(OA, "_causal_mask", lambda ts, Tq, Tk: np.ones((len(ts), Tk), dtype=bool))
    _assert_caught(_caught(["closed_forms", "causal_differs"]))


def test_scale_twice_caught(monkeypatch):
    orig = OA.dense_attention
    monkeypatch.setattr(oracle, "dense_attention",
                        lambda q, k, v, *, scale, **kw: orig(q, k, v, scale=scale * scale, **kw))
    _assert_caught(_caught(["brute_dense", "library_dense"]))


def test_lse_base2_caught(monkeypatch):
    orig = OA.dense_attention

    def log2_lse(*a, **kw):
        o, l = orig(*a, **kw)
        return o, l / math.log(2.0)

    monkeypatch.setattr(oracle, "dense_attention", log2_lse)
    _assert_caught(_caught(["library_dense", "lse_logsumexp"]))


def test_sparse_value_columns_caught(monkeypatch):
    monkeypatch.setattr(OA, "_value_rows", lambda G, d_v: G[:, G.shape[1] - d_v:][:, ::-1])
    _assert_caught(_caught(["brute_sparse", "sparse_equals_dense_mqa"]))


def test_window_ignored_caught(monkeypatch):
    monkeypatch.setattr(OA, "_window_mask", lambda ts, Tq, Tk, left, right: np.ones((len(ts), Tk), dtype=bool))
    _assert_caught(_caught(["window"]))


def test_window_rewrites_causal_caught(monkeypatch):
    """The defect the ArcFlash page names: a window clamp that turns causal into full attention."""
    orig = OA.dense_attention

    def clamp(q, k, v, *, causal, window=(-1, -1), **kw):
        return orig(q, k, v, causal=causal and window == (-1, -1), window=window, **kw)

    monkeypatch.setattr(oracle, "dense_attention", clamp)
    _assert_caught(_caught(["window"]))


def test_varlen_mask_dropped_caught(monkeypatch):
    """The varlen defect the ArcFlash page names: causal silently off for packed sequences."""
    orig = OA.dense_attention_varlen

    def non_causal(q, k, v, cu_q, cu_k, *, causal, **kw):
        return orig(q, k, v, cu_q, cu_k, causal=False, **kw)

    monkeypatch.setattr(oracle, "dense_attention_varlen", non_causal)
    _assert_caught(_caught(["varlen"]))


def test_two_part_rope_head_caught(monkeypatch):
    """Two-part rows with the rope key of kv head 0 used for every kv head."""
    orig = OA.dense_attention_two_part

    def head0(qn, qr, kn, kr, v, **kw):
        return orig(qn, qr, kn, np.asarray(kr, dtype=np.float64)[:, :1], v, **kw)

    monkeypatch.setattr(oracle, "dense_attention_two_part", head0)
    _assert_caught(_caught(["two_part"]))


def test_two_part_rope_dropped_caught(monkeypatch):
    """Two-part rows with the rope part left out of the scores."""
    def no_rope(qn, qr, kn, kr, v, **kw):
        return OA.dense_attention(qn, kn, v, **kw)

    monkeypatch.setattr(oracle, "dense_attention_two_part", no_rope)
    _assert_caught(_caught(["two_part"]))


def test_extras_sink_in_row_max_caught(monkeypatch):
    """The row maximum taken over the scores and the sink."""
    orig = OA.dense_attention_extras

    def with_sink(q, k, *, sinks=None, **kw):
        P, M = orig(q, k, sinks=sinks, **kw)
        if sinks is not None:
            M = np.maximum(M, np.asarray(sinks, dtype=np.float64)[None, :, None])
        return P, M

    monkeypatch.setattr(oracle, "dense_attention_extras", with_sink)
    _assert_caught(_caught(["extras"]))


def test_extras_rows_renormalised_caught(monkeypatch):
    """Probabilities renormalised to sum to 1, dropping the sink's share."""
    orig = OA.dense_attention_extras

    def renorm(q, k, **kw):
        P, M = orig(q, k, **kw)
        tot = P.sum(axis=-1, keepdims=True)
        return np.where(tot > 0, P / np.where(tot > 0, tot, 1.0), 0.0), M

    monkeypatch.setattr(oracle, "dense_attention_extras", renorm)
    _assert_caught(_caught(["extras"]))


def test_dropout_ignored_caught(monkeypatch):
    """The TransformerEngine page's review: dropout_p configured but not applied."""
    orig = OA.dense_attention

    def ignored(*a, keep=None, p_drop=0.0, **kw):
        return orig(*a, **kw)

    monkeypatch.setattr(oracle, "dense_attention", ignored)
    _assert_caught(_caught(["dropout"]))
