"""CPU oracle for head-heterogeneous block-sparse attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
"""
from .s2_oracle import (BLOCK, active_blocks, attend_keys, attn_bwd_dense, attn_decode, attn_decode_rows,
                        attn_fwd_blocks, block_minmax, block_minmax_paged, block_scores, select_blocks, attn_fwd_varlen, attn_fwd_dense, build_layout, dense_kv_blocks, paged_kv_blocks,
                        row_blocks, token_mask, transpose_layout)

__all__ = ["BLOCK", "active_blocks", "attend_keys", "attn_bwd_dense", "attn_decode", "attn_decode_rows",
           "block_minmax", "block_minmax_paged", "block_scores", "select_blocks",
           "attn_fwd_blocks", "attn_fwd_varlen", "attn_fwd_dense", "build_layout", "dense_kv_blocks", "paged_kv_blocks", "row_blocks",
           "token_mask", "transpose_layout"]
