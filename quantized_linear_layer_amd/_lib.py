"""ctypes declarations of libfp4lin.so (the C ABI in include/fp4lin.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4lin.so")

c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_ptr = ctypes.c_void_p
c_dbl = ctypes.c_double
c_int = ctypes.c_int

# enum values of fp4lin_status / fp4lin_dtype
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_QUANTILE, ERR_CAPACITY, ERR_ALIGN, ERR_WORKSPACE, \
    ERR_LAUNCH, ERR_SCRATCH = range(10)
F32, BF16 = 0, 1


class Coo(ctypes.Structure):
    _fields_ = [("row", c_ptr), ("col", c_ptr), ("val", c_ptr), ("row_ptr", c_ptr),
                ("capacity", c_i64)]


class ForwardOffsets(ctypes.Structure):
    _fields_ = [("tau", c_size), ("coo_row", c_size), ("coo_col", c_size), ("coo_val", c_size),
                ("row_ptr", c_size), ("Aq", c_size), ("sA", c_size), ("Wq", c_size),
                ("sW", c_size), ("scratch", c_size), ("capacity", c_i64), ("total", c_size)]


# name -> (restype, argtypes); every symbol declared in include/fp4lin.h
SIGNATURES = {
    "fp4lin_quantile_rank": (c_i64, [c_i64, c_dbl]),
    "fp4lin_packed_ld": (c_i64, [c_i64]),
    "fp4lin_select_workspace_bytes": (c_size, [c_i64, c_i64, c_int]),
    "fp4lin_weight_workspace_bytes": (c_size, [c_i64, c_i64]),
    "fp4lin_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_int, c_dbl]),
    "fp4lin_forward_layout": (c_int, [c_i64, c_i64, c_i64, c_int, c_dbl,
                                      ctypes.POINTER(ForwardOffsets)]),
    "fp4lin_status_str": (ctypes.c_char_p, [c_int]),
    "fp4lin_last_hip_error": (c_int, []),
    "fp4lin_last_hip_error_name": (ctypes.c_char_p, []),
    "fp4lin_outlier_select": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_dbl, c_ptr, Coo,
                                      c_ptr, c_size, c_ptr]),
    "fp4lin_outlier_select_noalloc": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_dbl, c_ptr,
                                              Coo, c_ptr]),
    "fp4lin_quantize_act": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr,
                                    c_ptr]),
    "fp4lin_quantize_weight": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr,
                                       c_size, c_ptr]),
    "fp4lin_gemm": (c_int, [c_ptr, c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64,
                            ctypes.POINTER(Coo), c_ptr, c_int, c_i64, c_ptr, c_i64, c_ptr]),
    "fp4lin_sparse_add": (c_int, [ctypes.POINTER(Coo), c_ptr, c_int, c_i64, c_i64, c_i64, c_i64,
                                  c_ptr, c_i64, c_ptr]),
    "fp4lin_forward": (c_int, [c_ptr, c_ptr, c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl,
                               c_ptr, c_i64, c_ptr, c_size, c_ptr]),
    "fp4lin_mx_scales_ld": (c_i64, [c_i64]),
    "fp4lin_quantize_act_mx": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_ptr,
                                       c_ptr]),
    "fp4lin_quantize_weight_mx": (c_int, [c_ptr, c_int, c_i64, c_i64, c_i64, c_ptr, c_ptr,
                                          c_ptr]),
    "fp4lin_gemm_mx": (c_int, [c_ptr, c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64,
                               ctypes.POINTER(Coo), c_ptr, c_int, c_i64, c_ptr, c_i64, c_ptr]),
    "fp4lin_workspace_bytes_mx": (c_size, [c_i64, c_i64, c_i64, c_int, c_dbl]),
    "fp4lin_forward_layout_mx": (c_int, [c_i64, c_i64, c_i64, c_int, c_dbl,
                                         ctypes.POINTER(ForwardOffsets)]),
    "fp4lin_forward_mx": (c_int, [c_ptr, c_ptr, c_int, c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl,
                                  c_ptr, c_i64, c_ptr, c_size, c_ptr]),
}

_lib = None


def load():
    """Load libfp4lin.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_linear_layer_amd.build` "
            "(there is no fallback implementation)")
    # PyTorch-ROCm ships its own HIP runtime with the same soname as the
    # system one the library is linked against. Loading torch first makes the
    # library bind to the runtime torch already holds, so both share one HIP
    # context; loaded the other way round, the process ends up with two
    # runtimes and the library's launches fail with hipErrorNoDevice.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
