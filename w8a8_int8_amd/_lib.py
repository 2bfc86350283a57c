"""ctypes loader of libw8a8.so and the prototypes of its C ABI (include/w8a8.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw8a8.so")

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t

# name -> (restype, argtypes); pointers and streams travel as void*
PROTOTYPES = {
    "w8a8_abi_version": (c_int, []),
    "w8a8_status_str": (ctypes.c_char_p, [c_int]),
    "w8a8_channel_amax": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp]),
    "w8a8_smooth_factors": (c_int, [c_vp, c_vp, c_i64, ctypes.c_double, c_vp, c_vp, c_vp]),
    "w8a8_calibrate_smooth_scratch_bytes": (c_size, [c_i64]),
    "w8a8_calibrate_smooth": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, ctypes.c_double,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "w8a8_calibrate_smooth_layers": (c_int, [c_vp, c_int, c_int, c_vp]),
    "w8a8_scale_quant_rows": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "w8a8_scale_quant_pair": (c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp,
                                      c_int, c_i64, c_vp]),
    "w8a8_fold_norm_weight": (c_int, [c_vp, c_vp, c_i64, c_vp, c_vp]),
    "w8a8_rmsnorm_quant_rows": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, ctypes.c_float, c_vp, c_vp,
                                        c_vp]),
    "w8a8_layernorm_quant_rows": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, ctypes.c_float,
                                          c_vp, c_vp, c_vp]),
    "w8a8_gemm_i32": (c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp]),
    "w8a8_gemm_dequant": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp]),
    "w8a8_scale_quant_rows_e4m3": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "w8a8_gemm_dequant_e4m3": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64,
                                       c_vp]),
    "w8a8_gemm_float": (c_int, [c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_vp]),
    "w8a8_linear_workspace_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "w8a8_linear": (c_int, [c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_size,
                            c_vp]),
    "w8a8_linear_noalloc": (c_int, [c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp]),
}

ABI_VERSION = 7
W8A8_F16, W8A8_BF16 = 0, 1



class CalibLayer(ctypes.Structure):
    """w8a8_calib_layer_t (include/w8a8.h): one entry of w8a8_calibrate_smooth_layers."""
    _fields_ = [("x_cal", c_vp), ("cal_rows", c_i64), ("w", c_vp), ("N", c_i64), ("K", c_i64),
                ("alpha", ctypes.c_double), ("amax_x", c_vp), ("amax_w", c_vp), ("s", c_vp),
                ("inv_s", c_vp), ("scratch", c_vp), ("scratch_bytes", c_size)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libw8a8.so from the package directory; fail loudly if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m w8a8_int8_amd.build). "
            "There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.w8a8_abi_version() != ABI_VERSION:
        raise ImportError(f"libw8a8 ABI {lib.w8a8_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
    return lib


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().w8a8_status_str(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise W8A8Error(fn, status)
