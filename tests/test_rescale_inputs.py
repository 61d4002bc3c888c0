"""The wide-dynamic-range inputs of tests/test_gpu_rescale.py do what they are for.

A kernel with a lazy online softmax moves its running maximum m only when a
key block's largest score exceeds m by more than 8 log2 units. These CPU
checks replay that rule over the score matrix of each input (numpy, block by
block in the order the kernels visit keys) and require that it fires after a
row's first visible block for a good share of the rows, at every block size
the kernels use (32, 64 and 128 keys). Without this, the GPU tests could pass
while the rescale branch never ran.
"""
import math

import numpy as np
import pytest

import oracle
import synth

LOG2E = 1.4426950408889634
THRESH = 8.0


def late_moves(S2: np.ndarray, bn: int) -> np.ndarray:
    """Per row of S2 (scores in log2 units, -inf where masked): how often the lazy
    maximum moves after the row's first block with a visible key."""
    R, n = S2.shape
    nb = (n + bn - 1) // bn
    pad = np.full((R, nb * bn), -np.inf)
    pad[:, :n] = S2
    bmax = pad.reshape(R, nb, bn).max(axis=2)
    m = np.full(R, -np.inf)
    moves = np.zeros(R, dtype=np.int64)
    for j in range(nb):
        x = bmax[:, j]
        started = np.isfinite(m)
        grow = started & (x - np.where(started, m, 0.0) > THRESH)
        moves += grow
        m = np.where(grow | (~started & np.isfinite(x)), x, m)
    return moves


def dense_scores(q, k, scale, causal):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, H, Tq, _ = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = H // Hkv
    rows = []
    for b in range(B):
        for h in range(H):
            S = scale * LOG2E * (q[b, h] @ k[b, h // g].T)
            if causal:
                S = np.where(np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + (Tk - Tq), S, -np.inf)
            rows.append(S)
    return np.concatenate(rows, axis=0)


def sparse_scores(q, pool, idx, scale):
    q, pool = np.asarray(q, np.float64), np.asarray(pool, np.float64)
    idx = np.asarray(idx)
    return np.concatenate([scale * LOG2E * (q[s] @ pool[idx[s]].T) for s in range(q.shape[0])], axis=0)


def _f64(t):
    return t.double().numpy()


def _assert_fires(S2, what, min_share):
    for bn in (32, 64, 128):
        moves = late_moves(S2, bn)
        share = float((moves > 0).mean())
        assert share >= min_share, f"{what}: the maximum moved after the first block in {share:.1%} of rows (bn={bn})"


# the least share of rows that must see a late move, per mode: "jump" moves
# only rows that see the late key (causal: the last seventh or so)
MIN_SHARE = {"qx16": 0.05, "rising": 0.3, "jump": 0.1}


@pytest.mark.parametrize("mode", synth.WIDE_MODES)
@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)])
def test_dense_inputs_move_the_maximum(dqk, dv, mode):
    inp = synth.widen_dense(1, 8, 2, 300, 300, dqk, dv, mode, sinks=False, seed=dqk + dv + len(mode))
    S2 = dense_scores(_f64(inp["q"]), _f64(inp["k"]), 1 / math.sqrt(dqk), True)
    _assert_fires(S2, f"dense d{dqk} {mode}", MIN_SHARE[mode])


@pytest.mark.parametrize("mode", synth.WIDE_MODES)
def test_decode_inputs_move_the_maximum(mode):
    inp = synth.widen_dense(1, 64, 1, 1, 3000, 512, 512, mode, sinks=True, seed=3000 + 512)
    S2 = dense_scores(_f64(inp["q"]), _f64(inp["k"]), 1 / math.sqrt(512), True)
    _assert_fires(S2, f"decode {mode}", 0.9 if mode != "qx16" else 0.05)


@pytest.mark.parametrize("mode", synth.WIDE_MODES)
def test_sparse_inputs_move_the_maximum(mode):
    inp = synth.widen_sparse(4, 64, 3000, 512, 300, mode, seed=3300)
    S2 = sparse_scores(_f64(inp["q"]), _f64(inp["kv"]), inp["idx"].numpy(), 1 / math.sqrt(512))
    _assert_fires(S2, f"sparse {mode}", 0.9 if mode != "qx16" else 0.05)


@pytest.mark.parametrize("mode", synth.WIDE_MODES)
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("shape", [(2, 8, 2, 3, 1500), (1, 32, 1, 2, 1500)], ids=["gqa12rows", "mqa64rows"])
def test_quantized_inputs_move_the_maximum(fmt, mode, shape):
    B, H, Hkv, Tq, Tk = shape
    inp = synth.widen_quant_kv(B, H, Hkv, Tq, Tk, 128, fmt, mode, sinks=True, seed=77)
    kd = oracle.dequantize_rows(inp["k"], fmt)
    S2 = dense_scores(_f64(inp["q"]), kd, 1 / math.sqrt(128), True)
    _assert_fires(S2, f"qkv {fmt} {mode}", 0.9 if mode != "qx16" else 0.05)


@pytest.mark.parametrize("mode", synth.WIDE_MODES)
def test_fp8_inputs_move_the_maximum(mode):
    inp = synth.widen_sparse_fp8(3, 64, 5000, 512, 2048, mode, sinks=True, seed=91)
    pool = oracle.dequantize_fp8_rows(inp["codes"].numpy(), inp["scales"].numpy())
    S2 = sparse_scores(_f64(inp["q"]), pool, inp["idx"].numpy(), 1 / math.sqrt(512))
    _assert_fires(S2, f"fp8 {mode}", 0.9 if mode != "qx16" else 0.05)


def test_late_moves_rule():
    """The replayed rule itself: a row whose block maxima climb 0, 5, 14, 30 (log2)
    moves at the third and fourth block only; a masked first block does not count."""
    S2 = np.array([[0.0, 5.0, 14.0, 30.0], [-np.inf, 0.0, 7.0, 9.0]])
    assert late_moves(S2, 1).tolist() == [2, 1]
