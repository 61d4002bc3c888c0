"""The ArcFlash page's memory arithmetic, reproduced from the shape.

Reading (stated in the design notes): scores and probabilities are both bf16
and each is bounded by the 32 MiB budget, so one tile holds
floor(32 MiB / (T * 2 B)) folded query rows; the tiled path's working set is
those two buffers plus the folded query tile and the unexpanded K and V. The
old path expands K and V to all 64 heads and materialises full bf16 scores
and probabilities. The page prints whole MiB, so each figure must agree to
within 1 MiB (the ratio to within 0.05).
"""
import os

import oracle

MIB = 1 << 20
HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    rows = {}
    with open(os.path.join(HERE, "golden", "arcflash_memory_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line or line.startswith("shape"):
                continue
            parts = line.split()
            rows[parts[0]] = [None if p == "-" else float(p) for p in parts[1:]]
    return rows


def test_arcflash_memory_table():
    g = _golden()
    H, T, D, e = 64, 1400, 512, 2
    budget = 32 * MIB
    rows = oracle.tile_rows_for_budget(budget, T, e)
    assert rows == 11983
    # the shape must really tile, with tiles straddling heads (folded rows = H*T)
    n_tiles = -(-H * T // rows)
    assert n_tiles == 8 and rows % T != 0
    expansion_old = 2 * H * T * D * e / MIB
    scores_old = 2 * H * T * T * e / MIB
    scores_new = 2 * rows * T * e / MIB
    qtile_kv_new = (rows * D * e + 2 * T * D * e) / MIB
    peak_old = expansion_old + scores_old
    peak_new = scores_new + qtile_kv_new
    assert abs(expansion_old - g["gqa_expansion_kv"][0]) <= 1
    assert g["gqa_expansion_kv"][1] == 0
    assert abs(scores_old - g["score_matrices"][0]) <= 1
    assert abs(scores_new - g["score_matrices"][1]) <= 1
    assert abs(qtile_kv_new - g["folded_query_tile_kv"][1]) <= 1
    assert abs(peak_old - g["peak"][0]) <= 1
    assert abs(peak_new - g["peak"][1]) <= 1
    assert abs(peak_old / peak_new - g["ratio"][0]) <= 0.05
