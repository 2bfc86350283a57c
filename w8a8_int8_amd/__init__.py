"""SmoothQuant W8A8 linear-layer path for MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libw8a8.so`` (built by ``w8a8_int8_amd.build``); this
package only marshals torch tensors into its C entry points.
"""
from .api import (calibrate_smooth, calibrate_smooth_layers, calibrate_smooth_scratch, channel_amax, fold_layernorm,
                  fold_norm_weight, gemm_dequant, gemm_dequant_e4m3, gemm_float, gemm_i32,
                  layernorm_quant_rows, linear, linear_noalloc, linear_workspace_bytes,
                  prepare_weight,
                  rmsnorm_quant_rows, scale_quant_pair, scale_quant_rows, scale_quant_rows_e4m3,
                  smooth_factors)

__all__ = [
    "channel_amax", "smooth_factors", "scale_quant_rows", "scale_quant_pair", "gemm_i32",
    "gemm_dequant", "gemm_float", "linear", "linear_noalloc", "linear_workspace_bytes", "prepare_weight",
    "scale_quant_rows_e4m3", "gemm_dequant_e4m3", "fold_norm_weight", "rmsnorm_quant_rows",
    "fold_layernorm", "layernorm_quant_rows", "calibrate_smooth", "calibrate_smooth_layers",
    "calibrate_smooth_scratch",
]
