"""ctypes loader of libi8mm.so (argument types only; no computation here)."""

from __future__ import annotations

import ctypes
import os
import re
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libi8mm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "i8mm.h")

c_i64 = ctypes.c_int64
c_p = ctypes.c_void_p
c_f = ctypes.c_float
c_int = ctypes.c_int
c_size = ctypes.c_size_t

_SIGNATURES = {
    "i8mm_quantize_colwise_weights": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p]),
    "i8mm_detect_outlier_cols": (c_int, [c_p, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p]),
    "i8mm_quantize_rowwise": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_p]),
    "i8mm_int8_mixed_matmul": (c_int, [c_p, c_p, c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_p,
                                       c_i64, c_i64, c_i64, c_p, c_p]),
    "i8mm_outlier_matmul": (c_int, [c_p, c_i64, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_p, c_p]),
    "i8mm_int8_gemm_i32": (c_int, [c_p, c_p, c_i64, c_i64, c_i64, c_p, c_p]),
    "i8mm_pack_fp16_weights": (c_int, [c_p, c_i64, c_i64, c_p, c_p]),
    "i8mm_fp16_gemm": (c_int, [c_p, c_p, c_i64, c_i64, c_i64, c_p, c_p]),
    "i8mm_quantize_tensorwise": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_p]),
    "i8mm_quantize_weights_tensorwise": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p]),
    "i8mm_quantize_rowwise_zeropoint": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                                c_p, c_i64, c_p]),
    "i8mm_quantize_colwise_weights_zeropoint": (c_int, [c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_zeropoint_matmul": (c_int, [c_p, c_p, c_p, c_p, c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                      c_i64, c_i64, c_i64, c_p, c_p]),
    "i8mm_forward_workspace_bytes": (c_size, [c_i64, c_i64]),
    "i8mm_forward": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_forward_workspace_layout": (c_int, [c_i64, c_i64, ctypes.POINTER(c_size), ctypes.POINTER(c_i64)]),
    "i8mm_forward_tensorwise": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_forward_zeropoint_workspace_bytes": (c_size, [c_i64, c_i64]),
    "i8mm_forward_zeropoint": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                       c_p]),
    "i8mm_forward_decode": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_forward_inline_quant": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_forward_noalloc": (c_int, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p, c_p, c_p, c_p, c_p]),
    "i8mm_calib_mfma_i8": (c_int, [c_p, c_i64, c_i64, c_p, c_p]),
    "i8mm_test_fail_product_launches": (None, [c_int]),
    "i8mm_version": (ctypes.c_char_p, []),
    "i8mm_status_string": (ctypes.c_char_p, [c_int]),
}

_lib = None


def header_functions(path: str = HEADER) -> List[str]:
    """Names of the functions declared in include/i8mm.h."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(i8mm_[a-z0-9_]+)\s*\(", text)))


def header_define(name: str, path: str = HEADER) -> int:
    """Integer value of a `#define name value` line of include/i8mm.h."""
    with open(path) as f:
        m = re.search(r"^#define\s+" + re.escape(name) + r"\s+(\d+)\s*$", f.read(), flags=re.M)
    if m is None:
        raise KeyError(name)
    return int(m.group(1))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libi8mm.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libi8mm.so not found at {path}: build it first with "
            "`python -m int8_quantized_matmul_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def loaded_path() -> str:
    return LIB_PATH
