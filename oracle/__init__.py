"""CPU oracle (test infrastructure only; never on the product path).

Only tests/, the smoke check in __graft_entry__.py and bench.py's CPU
baseline leg import this package.
"""
from .smoothquant import *  # noqa: F401,F403
from .smoothquant import (QMAX, apply_col_scale, channel_amax, dequant, gemm_float, gemm_i32,
                          linear, narrow, prepare_weight, quantize_rows,
                          round_to_bf16, scale_quant_rows, smooth_factor,
                          smooth_factors, smooth_fp64, widen)
from .smoothquant import (E4M3_MAX, e4m3_to_float, e4m3_value, gemm_e4m3,
                          quantize_rows_e4m3, round_to_e4m3, scale_quant_rows_e4m3)
from .smoothquant import fold_norm_weight, rms_inv, rmsnorm_fp64, rmsnorm_smooth_quant_rows
from .smoothquant import layernorm_fp64, layernorm_smooth_quant_rows, layernorm_stats
