"""Grouped block-scaled (MX) GEMM for MoE expert layers on AMD MI355X (gfx950).

The compute path is libmxgg.so (hand-written HIP kernels behind the C ABI of
include/mxgg.h); this package is its thin ctypes binding.
"""
from ._lib import (  # noqa: F401
    FORMATS, FP8_1x128, FP8_128x128, FP8_1x128_P2, FP8_128x128_P2, LAYOUT_BLOCK_MAJOR, LAYOUT_MASK, LAYOUT_MFMA,
    LAYOUT_ROW_MAJOR, KBLOCK_COLS, KBLOCK_MASK, KBLOCK_ROWS,
    LIB_PATH, MAX_EXPERTS, MXFP4, MXFP8, POW2_SCALES,
    MxggError, header_functions, lib,
    mxgg_grouped_dgrad, mxgg_grouped_fwd, mxgg_grouped_wgrad, mxgg_quantize_colwise_segpad, mxgg_quantize_dual,
    mxgg_mx_scale_stride, mxgg_mx_scales_relayout, mxgg_quantize_rowwise, mxgg_segpad_rows, mxgg_transpose_128x128,
    mxgg_workspace_size,
    grouped_dgrad, grouped_fwd, grouped_wgrad, quantize_colwise_segpad, quantize_dual, quantize_rowwise,
    mx_scale_stride, mx_scales_relayout, segpad_rows, transpose_128x128, workspace_size,
)
