"""fp64 CPU oracle for the attention forward and backward -- test infrastructure only.

Importable by the tests, the package smoke check and the bench's CPU-baseline
leg; never by the product path.
"""
from .attention import (  # noqa: F401
    dense_attention,
    dense_attention_backward,
    dense_attention_extras,
    dense_attention_tiled,
    dense_attention_two_part,
    dense_attention_varlen,
    decode_fp8_e4m3,
    dequantize_fp8_rows,
    dequantize_rows,
    gather_rows,
    merge_partials,
    repeat_kv,
    scatter_add_rows,
    sparse_topk_attention,
    sparse_topk_attention_backward,
    sum_kv_groups,
    tile_rows_for_budget,
)
