"""Plain CPU oracle of the quantiser variants the pages compare with
vector-wise absmax (TEST INFRASTRUCTURE ONLY, like the rest of oracle/:
nothing on the product path may import, call or run it).

[DIGEST] "Quantization Primitives: Absmax and Zeropoint Quantization" and
"Vector-wise Quantization" (Table 1's hierarchy: tensor-wise absmax,
row-wise absmax with one tensor-wide constant for W, vector-wise, and
zeropoint vector-wise, each also with the mixed-precision decomposition);
[PY] "量化为什么会崩：一个尺度统治全局" (the zero point and the four-term product on GPUs;
row-wise and vector-wise granularity); [TM] "Absmax INT8
quantization from first principles".

Every variant keeps the decomposition of the main path: the outlier columns
O (from llm_int8.outlier_columns) leave the 8-bit part and are multiplied in
16 bit; with alpha = inf there is no decomposition. Precision follows the
main oracle: fp32 scales from one IEEE division, one fp32 multiply before
rounding half away from zero, exact integer products, the fp16 output
rounded once from a float64 sum.

Readings (the pages leave these open or print them garbled):
  * tensor-wise: one absmax over the whole non-outlier part of the tensor
    (all rows, all columns not in O); the constant is returned broadcast,
    c_x [s] (or c_w [o]) with every entry equal, so the product is the
    vector-wise one with equal constants.
  * zeropoint: nd = fl32(254 / fl32(max - min)) over the row of X (the
    column of W), min and max taken over the values themselves (signed) and,
    for X, over the columns not in O. The zero point's printed formula
    (X times min) is garbled; read as zp = round(fl32(nd * min)) + 127, so
    the codes q = round(fl32(nd * x)) - zp, clamped to [-127, 127], span the
    whole range and q + zp approximates nd * x: the form in which the
    four-term product adds the zero points back. zp is an integer that can
    leave int16 for one-signed data (the pages' i16 suffix) and is kept in
    int32. A row or column with max == min gets nd = 1.
  * the zeropoint product runs over the non-outlier columns only:
    C'_ij = sum_{k not in O} (Xq_ik + zp_x_i) (Wq_kj + zp_w_j), exact, and
    C = fp16(C' / (nd_x_i nd_w_j) + C^O [+ b]).
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .llm_int8 import dequantize_and_add, int8_matmul_i32, outlier_matmul, round_half_away, row_scales

__all__ = [
    "quantize_tensorwise",
    "quantize_weights_tensorwise",
    "zeropoint_params",
    "quantize_rowwise_zeropoint",
    "quantize_colwise_weights_zeropoint",
    "zeropoint_product_i64",
    "zeropoint_matmul",
    "variant_forward",
]

F32 = np.float32
F64 = np.float64


def _regular(h: int, idx: np.ndarray) -> np.ndarray:
    reg = np.ones(h, dtype=bool)
    reg[np.asarray(idx, dtype=np.int64)] = False
    return reg


def quantize_tensorwise(X_f16: np.ndarray, idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Tensor-wise absmax for X ([DIGEST] "Quantization Primitives": one
    scaling constant 127 / ||X||_inf for the whole tensor), over the columns
    not in O. Returns Xq int8 [s, h] (O columns 0), c_x fp32 [s] (all equal),
    X_O fp16 [s, |O|]."""
    X16 = np.asarray(X_f16, dtype=np.float16)
    s, h = X16.shape
    reg = _regular(h, idx)
    X32 = X16.astype(F32)
    m = np.abs(X32[:, reg]).max() if reg.any() and s > 0 else F32(0.0)
    c = row_scales(np.array([m], dtype=F32))[0]
    v = (X32 * c).astype(F32)
    q = np.clip(round_half_away(v), -127, 127)
    q[:, ~reg] = 0
    return q.astype(np.int8), np.full(s, c, dtype=F32), X16[:, np.asarray(idx, dtype=np.int64)].copy()


def quantize_weights_tensorwise(W_f16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Tensor-wise absmax for W (load time): one constant 127 / ||W||_inf.
    Used by both tensor-wise and row-wise quantisation ([DIGEST]
    "Vector-wise Quantization": row-wise keeps row constants for X and a
    single tensor-wise constant for W). Returns Wq_t int8 [o, h], c_w [o]
    (all equal)."""
    W32 = np.asarray(W_f16, dtype=np.float16).astype(F32)
    h, o = W32.shape
    m = np.abs(W32).max() if W32.size else F32(0.0)
    c = row_scales(np.array([m], dtype=F32))[0]
    q = np.clip(round_half_away((W32 * c).astype(F32)), -127, 127).astype(np.int8)
    return np.ascontiguousarray(q.T), np.full(o, c, dtype=F32)


def zeropoint_params(lo: np.ndarray, hi: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Zeropoint constants of [DIGEST] "Quantization Primitives" for vectors
    of minima and maxima: nd = fl32(254 / fl32(hi - lo)) (the normalised
    dynamic range, twice 127 over the span; 1 where hi == lo) and
    zp = round(fl32(nd * lo)) + 127 (int64; reading in the module
    docstring)."""
    lo = np.asarray(lo, dtype=F32)
    hi = np.asarray(hi, dtype=F32)
    span = (hi - lo).astype(F32)                                # one fp32 rounding
    nd = np.where(span > 0, (F32(254.0) / np.where(span > 0, span, F32(1.0))).astype(F32), F32(1.0)).astype(F32)
    zp = round_half_away((nd * lo).astype(F32)).astype(np.int64) + 127
    return nd, zp


def _zp_codes(x32: np.ndarray, nd: np.ndarray, zp: np.ndarray) -> np.ndarray:
    """q = clamp(round(fl32(nd x)) - zp, -127, 127) (nd, zp broadcast)."""
    v = (x32 * nd).astype(F32)
    return np.clip(round_half_away(v) - zp, -127, 127)


def quantize_rowwise_zeropoint(X_f16: np.ndarray, idx: np.ndarray
                               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Zeropoint quantisation of each row of X over the columns not in O.
    Returns Xq int8 [s, h] (O columns 0), nd_x fp32 [s], zp_x int32 [s],
    X_O fp16 [s, |O|]."""
    X16 = np.asarray(X_f16, dtype=np.float16)
    s, h = X16.shape
    reg = _regular(h, idx)
    X32 = X16.astype(F32)
    if reg.any():
        lo, hi = X32[:, reg].min(axis=1), X32[:, reg].max(axis=1)
    else:
        lo = hi = np.zeros(s, dtype=F32)
    nd, zp = zeropoint_params(lo, hi)
    q = _zp_codes(X32, nd[:, None], zp[:, None])
    q[:, ~reg] = 0
    return q.astype(np.int8), nd, zp.astype(np.int32), X16[:, np.asarray(idx, dtype=np.int64)].copy()


def quantize_colwise_weights_zeropoint(W_f16: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Zeropoint quantisation of each column of W over all h rows (load
    time). Returns Wq_t int8 [o, h], nd_w fp32 [o], zp_w int32 [o]."""
    W32 = np.asarray(W_f16, dtype=np.float16).astype(F32)
    nd, zp = zeropoint_params(W32.min(axis=0), W32.max(axis=0))
    q = _zp_codes(W32, nd[None, :], zp[None, :]).astype(np.int8)
    return np.ascontiguousarray(q.T), nd, zp.astype(np.int32)


def zeropoint_product_i64(Xq: np.ndarray, zp_x: np.ndarray, Wq_t: np.ndarray, zp_w: np.ndarray,
                          idx: np.ndarray) -> np.ndarray:
    """C'_ij = sum over k not in O of (Xq_ik + zp_x_i)(Wq_kj + zp_w_j), exact
    in int64: the product of the zero-point-shifted codes ([DIGEST]
    "Quantization Primitives", the product of two zeropoint-quantised
    matrices; [PY] "量化为什么会崩：一个尺度统治全局"), taken as written, not expanded."""
    h = Xq.shape[1]
    reg = _regular(h, idx)
    A = Xq[:, reg].astype(np.int64) + np.asarray(zp_x, dtype=np.int64)[:, None]
    B = Wq_t[:, reg].astype(np.int64) + np.asarray(zp_w, dtype=np.int64)[:, None]
    return A @ B.T


def zeropoint_matmul(Xq, nd_x, zp_x, X_O, idx, Wq_t, nd_w, zp_w, W_f16,
                     bias: Optional[np.ndarray] = None, col_chunk: int = 4096) -> np.ndarray:
    """C = fp16( C' / (nd_x (x) nd_w) + X_O W[O, :] [+ b] ): the zeropoint
    vector-wise product with the 16-bit outlier part of the decomposition
    ([DIGEST] "Mixed-Precision Decomposition"; Table 1's zeropoint rows).
    C' is exact (int64); its conversion to float64 is exact below 2^53."""
    s = Xq.shape[0]
    o = Wq_t.shape[0]
    C = np.empty((s, o), dtype=np.float16)
    for j0 in range(0, o, col_chunk):
        j1 = min(o, j0 + col_chunk)
        Cp = zeropoint_product_i64(Xq, zp_x, Wq_t[j0:j1], zp_w[j0:j1], idx)
        CO = outlier_matmul(X_O, W_f16[:, j0:j1], idx)
        # dequantize_and_add divides by the product of the two constants
        C[:, j0:j1] = dequantize_and_add(Cp, nd_x, nd_w[j0:j1], CO, None if bias is None else bias[j0:j1])
    return C


def variant_forward(X_f16: np.ndarray, W_f16: np.ndarray, scheme: str, alpha: float = 6.0,
                    bias: Optional[np.ndarray] = None) -> np.ndarray:
    """C for one quantiser scheme of Table 1, with the decomposition at
    threshold alpha (alpha = inf: none): "tensor" (tensor-wise X and W),
    "row" (row-wise X, tensor-wise W), "vector" (the main path) or
    "zeropoint" (zeropoint vector-wise)."""
    from .llm_int8 import outlier_columns, quantize_colwise_weights, quantize_rowwise
    _, idx, _ = outlier_columns(X_f16, alpha)
    if scheme == "zeropoint":
        Xq, nd_x, zp_x, X_O = quantize_rowwise_zeropoint(X_f16, idx)
        Wq_t, nd_w, zp_w = quantize_colwise_weights_zeropoint(W_f16)
        return zeropoint_matmul(Xq, nd_x, zp_x, X_O, idx, Wq_t, nd_w, zp_w, W_f16, bias=bias)
    if scheme == "tensor":
        Xq, c_x, X_O = quantize_tensorwise(X_f16, idx)
        Wq_t, c_w = quantize_weights_tensorwise(W_f16)
    elif scheme == "row":
        Xq, c_x, X_O = quantize_rowwise(X_f16, idx)
        Wq_t, c_w = quantize_weights_tensorwise(W_f16)
    elif scheme == "vector":
        Xq, c_x, X_O = quantize_rowwise(X_f16, idx)
        Wq_t, c_w = quantize_colwise_weights(W_f16)
    else:
        raise ValueError(f"unknown scheme {scheme!r}")
    Ci = int8_matmul_i32(Xq, Wq_t)
    CO = outlier_matmul(X_O, W_f16, idx)
    return dequantize_and_add(Ci, c_x, c_w, CO, bias)
