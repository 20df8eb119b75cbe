"""LoopVQ hot path for AMD Instinct MI355X: loop-axis VQ encoder and paged decode
attention over the coded KV cache, as HIP kernels behind a C ABI (include/lvq.h).

The binding lives in ``sub_bit_loop_amd._abi``; importing this package does not
load the library (that happens on first use and raises if it is not built).
"""
from ._abi import (  # noqa: F401
    AttnShape, CacheDesc, LvqError, PagedCache, ReencodeLayer, RowsShape, lib, lvq_build_codebooks,
    lvq_decode_attn, lvq_decode_attn_noalloc, lvq_decode_attn_workspace_bytes, lvq_decode_scores, lvq_encode, lvq_encode_pages,
    lvq_reencode_pages, lvq_reencode_pages_layers, lvq_rope_table_bytes, lvq_rope_tables, lvq_rows_attn,
    lvq_rows_attn_workspace_bytes, lvq_version, make_rows_shape, make_shape,
)
