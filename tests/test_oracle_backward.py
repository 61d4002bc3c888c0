"""The oracle's backward against finite differences, torch autograd, closed forms and
invariants; planted mistakes in it must each be caught (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import attention as OA
from tests import pins_bwd


@pytest.mark.parametrize("name", sorted(pins_bwd.ALL_CHECKS))
def test_backward_pin(name):
    err = pins_bwd.ALL_CHECKS[name]()
    assert err <= pins_bwd.TOL, f"{name}: discrepancy {err:.3e}"


def _assert_caught(names):
    results = {n: pins_bwd.ALL_CHECKS[n]() for n in names}
    assert any(v > pins_bwd.TOL for v in results.values()), f"mutation not caught: {results}"


def test_dropped_D_term_caught(monkeypatch):
    monkeypatch.setattr(OA, "_softmax_backward", lambda P, dP, dO, O: P * dP)
    _assert_caught(["bwd_finite_differences", "bwd_invariants"])


def test_wrong_sign_caught(monkeypatch):
    orig = OA._softmax_backward
    monkeypatch.setattr(OA, "_softmax_backward", lambda P, dP, dO, O: -orig(P, dP, dO, O))
    _assert_caught(["bwd_finite_differences", "bwd_library_autograd"])


def test_rep_major_head_sum_caught(monkeypatch):
    def rep_major(x, g):
        B, H, T, D = x.shape
        y = np.zeros((B, H // g, T, D))
        for kv in range(H // g):
            for rep in range(g):
                y[:, kv] += x[:, rep * (H // g) + kv]
        return y

    monkeypatch.setattr(OA, "sum_kv_groups", rep_major)
    _assert_caught(["bwd_finite_differences", "bwd_library_autograd"])


def test_missing_scale_caught(monkeypatch):
    orig = OA.dense_attention_backward

    def unscaled(q, k, v, dout, *, scale, **kw):
        dq, dk, dv, ds = orig(q, k, v, dout, scale=scale, **kw)
        return dq / scale, dk / scale, dv, ds

    monkeypatch.setattr(oracle, "dense_attention_backward", unscaled)
    _assert_caught(["bwd_finite_differences", "bwd_library_autograd"])


def test_sink_gradient_sign_caught(monkeypatch):
    orig = OA.dense_attention_backward

    def flipped(*a, **kw):
        dq, dk, dv, ds = orig(*a, **kw)
        return dq, dk, dv, (None if ds is None else -ds)

    monkeypatch.setattr(oracle, "dense_attention_backward", flipped)
    _assert_caught(["bwd_finite_differences", "bwd_library_autograd"])


def test_sparse_value_role_dropped_caught(monkeypatch):
    """The pool's gradient without its value-role term P^T dO."""
    orig = OA.sparse_topk_attention_backward

    def key_only(q, kv, idx, dout, *, d_v, scale, sinks=None):
        dq, dkv, ds = orig(q, kv, idx, dout, d_v=d_v, scale=scale, sinks=sinks)
        # subtract the value-role part again, recomputed per query
        qf, kvf, do = (np.asarray(x, np.float64) for x in (q, kv, dout))
        for s in range(qf.shape[0]):
            keep = [int(n) for n in idx[s] if 0 <= int(n) < kvf.shape[0]]
            Gm = kvf[keep]
            S = scale * (qf[s] @ Gm.T)
            m = S.max(axis=1, keepdims=True)
            if sinks is not None:
                m = np.maximum(m, np.asarray(sinks)[:, None])
            e = np.exp(S - m)
            den = e.sum(axis=1, keepdims=True) + (0 if sinks is None else np.exp(np.asarray(sinks)[:, None] - m))
            P = e / den
            contrib = P.T @ do[s]
            for j, n in enumerate(keep):
                dkv[n, :d_v] -= contrib[j]
        return dq, dkv, ds

    monkeypatch.setattr(oracle, "sparse_topk_attention_backward", key_only)
    _assert_caught(["sparse_bwd_finite_differences", "sparse_bwd_library_autograd"])


def test_sparse_duplicates_collapsed_caught(monkeypatch):
    """A scatter that overwrites instead of adding loses a duplicated index's second slot."""
    def assign(y, idx, rows):
        seen = {}
        for j, n in enumerate(idx):
            if 0 <= int(n) < y.shape[0]:
                seen[int(n)] = rows[j]       # the last slot wins: duplicates collapse
        for n, r in seen.items():
            y[n] += r

    monkeypatch.setattr(OA, "scatter_add_rows", assign)
    _assert_caught(["sparse_bwd_finite_differences"])


def test_dropout_mask_ignored_in_backward_caught(monkeypatch):
    """The TransformerEngine page's review: a backward that drops the dropout state
    while the forward applied it."""
    orig = OA.dense_attention_backward

    def no_mask(*a, keep=None, p_drop=0.0, **kw):
        return orig(*a, **kw)

    monkeypatch.setattr(oracle, "dense_attention_backward", no_mask)
    _assert_caught(["bwd_dropout"])
