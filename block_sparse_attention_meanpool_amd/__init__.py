"""Block-sparse attention with mean-pooled block selection on MI355X (gfx950).

The compute path is libsla.so (HIP kernels behind a C ABI, declared in
include/sla.h); this package is its Python binding.
"""

from .binding import (CLS_CRITICAL, CLS_MARGINAL, CLS_SKIP, EXPORTS, FLAG_BAD_CLASS, FLAG_OVERFLOW,
                      LIB_PATH, MODES, SlaAttention, SlaError, count_from_fraction, counts_for,
                      debug_flag_address, sla_check_lists, sla_check_row_order, sla_row_order,
                      sla_clock_probe, probe_clock_hz,
                      FLAG_LIST_RANGE, FLAG_LIST_REPEAT, FLAG_LIST_ORDER, FLAG_LIST_COUNT,
                      FLAG_ORDER_PERM,
                      forward, lib, num_blocks, sla_attention, sla_block_mask, sla_combine,
                      sla_dense_attn_fwd, sla_linear_branch_bwd, sla_linear_branch_fwd,
                      sla_linear_branch_prepare, sla_mask_recall, sla_pool_classify,
                      sla_pool_classify_noalloc,
                      sla_sparse_attn_bwd, sla_sparse_attn_fwd, sla_sparse_linear_attn_fwd,
                      sla_status_string, sla_tile_permute, sla_version)

__all__ = ["CLS_CRITICAL", "CLS_MARGINAL", "CLS_SKIP", "EXPORTS", "FLAG_BAD_CLASS", "FLAG_OVERFLOW",
           "LIB_PATH", "MODES", "SlaAttention", "SlaError", "count_from_fraction", "counts_for",
           "debug_flag_address", "sla_check_lists", "sla_check_row_order", "sla_row_order",
           "sla_clock_probe", "probe_clock_hz",
           "FLAG_LIST_RANGE", "FLAG_LIST_REPEAT", "FLAG_LIST_ORDER", "FLAG_LIST_COUNT",
           "FLAG_ORDER_PERM",
           "forward", "lib", "num_blocks", "sla_attention", "sla_block_mask", "sla_combine",
           "sla_dense_attn_fwd", "sla_linear_branch_bwd", "sla_linear_branch_fwd",
           "sla_linear_branch_prepare", "sla_mask_recall", "sla_pool_classify",
           "sla_pool_classify_noalloc",
           "sla_sparse_attn_bwd", "sla_sparse_attn_fwd", "sla_sparse_linear_attn_fwd",
           "sla_status_string", "sla_tile_permute", "sla_version"]
