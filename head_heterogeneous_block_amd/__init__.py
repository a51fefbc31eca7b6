"""MI355X (gfx950) head-heterogeneous block-sparse causal attention (S2-Attention / HHST).

The compute path is libs2attn.so (hand-written HIP kernels behind the C ABI in
include/s2attn.h); ``s2attn`` is its ctypes binding.
"""
from .s2attn import (S2_BLOCK, Layout, Pattern, PreparedBwd, PreparedDecode, PreparedDecodePaged,
                     PreparedFwd, PreparedFwdVarlen, s2_attn_fwd_varlen, PreparedLayout, S2Error, library, s2_abi_version, s2_attn_bwd,
                     s2_attn_bwd_workspace, s2_attn_decode, s2_attn_decode_paged,
                     s2_attn_decode_paged_workspace, s2_attn_decode_workspace, s2_attn_fwd,
                     s2_attn_fwd_workspace, s2_attn_decode_noalloc, s2_build_layout, s2_build_layout_t, s2_last_error, s2_layout_nnz, layout_from_csr,
                     s2_validate_layout, s2_transpose_layout, s2_transpose_layout_workspace,
                     PreparedSelectDecode, s2_attn_decode_rows, s2_attn_decode_rows_workspace, s2_block_minmax,
                     s2_select_blocks, PreparedSelectDecodePaged, s2_attn_decode_paged_rows,
                     s2_attn_decode_paged_rows_workspace, s2_block_minmax_paged)

__all__ = ["S2_BLOCK", "Layout", "Pattern", "PreparedBwd", "PreparedDecode", "PreparedDecodePaged",
           "PreparedFwd", "PreparedFwdVarlen", "s2_attn_fwd_varlen", "PreparedLayout", "S2Error", "library", "s2_abi_version", "s2_attn_bwd",
           "s2_attn_bwd_workspace", "s2_attn_decode", "s2_attn_decode_paged",
           "s2_attn_decode_paged_workspace", "s2_attn_decode_workspace", "s2_attn_fwd",
           "s2_attn_fwd_workspace", "s2_attn_decode_noalloc", "s2_build_layout", "s2_build_layout_t", "s2_last_error", "s2_layout_nnz", "layout_from_csr",
           "s2_validate_layout", "s2_transpose_layout", "s2_transpose_layout_workspace",
           "PreparedSelectDecode", "s2_attn_decode_rows", "s2_attn_decode_rows_workspace", "s2_block_minmax",
           "s2_select_blocks", "PreparedSelectDecodePaged", "s2_attn_decode_paged_rows",
           "s2_attn_decode_paged_rows_workspace", "s2_block_minmax_paged"]
