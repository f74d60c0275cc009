"""Plain CPU oracle of the LLM.int8() decomposed matrix multiply C = X W.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, header, table or helper with the
HIP implementation, and it is deliberately slow and obvious.

Page tags used in the citations:
  [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale"
           (paper-graph-ui.vercel.app digest of arXiv 2208.07339)
  [TM]     transformer-math tutorial on LLM.int8() (aicassindra.com)
  [PY]     "LLM.int8() 完全拆解：系统离群值的涌现与混合精度分解" (pinghaoyang.com.cn)

The method is an approximation with a fixed encoding, so the oracle takes the
steps of [DIGEST] "The Full LLM.int8() Algorithm" (Steps 1-5) in that order,
in the pages' notation: X_f16 [s, h], W_f16 [h, o], outlier set O, row scales
c_x [s], column scales c_w [o], C_i32, S = 1 / (c_x ⊗ c_w).

Precision (the pages say only "round to the nearest integer"; these readings
are fixed here and by the GPU path alike):
  * every fp16 input is widened to fp32 exactly;
  * comparisons with alpha are in fp32;
  * scales are fp32: c = fl32(127 / m), one IEEE round-to-nearest-even division;
    a zero absmax gives c = 1 (all quantised values are then 0);
  * quantisation is one fp32 multiply v = fl32(x * c) followed by rounding
    half away from zero, done exactly in float64, clamped to [-127, 127];
  * C_i32 is exact (a float64 product of int8-valued arrays: every partial
    sum is an integer below 2**53, so the result is exact in any order);
  * the outlier product and the dequantised sum are float64, rounded once to
    fp16 (round to nearest even).

Parity pins for every function live in tests/test_oracle_pins.py. Two choices
are conventions rather than page facts and are "parity unpinned": the scale
1.0 for an all-zero row/column, and c_w taken over all h rows of W (see
quantize_colwise_weights).
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "fp16_matmul",
    "dequantized_outlier_rows",
    "outlier_columns",
    "mask_from_indices",
    "row_scales",
    "quantize_rowwise",
    "quantize_colwise_weights",
    "int8_matmul_i32",
    "outlier_matmul",
    "dequantize_and_add",
    "int8_mixed_matmul",
    "forward",
    "round_half_away",
]

F32 = np.float32
F64 = np.float64


def round_half_away(v: np.ndarray) -> np.ndarray:
    """Round to nearest, ties away from zero, evaluated exactly in float64.

    [TM] "Absmax INT8 quantization from first principles": Q(x) = round(s x).
    Reading: ties go away from zero (the pages do not say which way ties go).
    ``v`` holds fp32 values, so |v| + 0.5 is exact in float64.
    """
    v64 = np.asarray(v, dtype=F64)
    return np.sign(v64) * np.floor(np.abs(v64) + 0.5)


def mask_from_indices(idx: np.ndarray, h: int) -> np.ndarray:
    """Bit j of word j // 32 is set iff column j is in O (little-endian bits)."""
    nwords = (h + 31) // 32
    mask = np.zeros(nwords, dtype=np.uint32)
    for j in np.asarray(idx, dtype=np.int64):
        mask[j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return mask


def outlier_columns(X_f16: np.ndarray, alpha: float = 6.0) -> Tuple[np.ndarray, np.ndarray, int]:
    """Step 1, outlier detection: O = { j in [0, h) : max_i |X_ij| >= alpha }.

    [DIGEST] "The Full LLM.int8() Algorithm", Step 1 (scan X column-wise, keep
    every feature dimension whose largest magnitude is at least 6.0);
    [DIGEST] "Mixed-Precision Decomposition", formal definition of O;
    [PY] "第二件武器：混合精度分解" (threshold alpha = 6.0).
    Readings: ">=" (the digest's wording) rather than "exceeds"; the index range
    is 0 <= j < h. A column is in O when some element of it reaches alpha,
    tested element by element, so a NaN elsewhere in the column neither adds
    nor removes it. Returns (mask u32[ceil(h/32)], idx int32 ascending, |O|).
    """
    X32 = np.asarray(X_f16, dtype=np.float16).astype(F32)
    s, h = X32.shape
    if s == 0:
        idx = np.zeros(0, dtype=np.int32)
    else:
        reaches = np.abs(X32) >= F32(alpha)          # False for NaN
        idx = np.nonzero(reaches.any(axis=0))[0].astype(np.int32)
    return mask_from_indices(idx, h), idx, int(idx.size)


def row_scales(m: np.ndarray) -> np.ndarray:
    """c = 127 / m in fp32 (one IEEE division); c = 1 where m == 0.

    [TM] "Absmax INT8 quantization from first principles": s = 127 / absmax(x);
    [DIGEST] "Vector-wise Quantization": c_x_i = 127 / max_j |X_ij|.
    """
    m = np.asarray(m, dtype=F32)
    safe = np.where(m > 0, m, F32(1.0)).astype(F32)
    c = (F32(127.0) / safe).astype(F32)
    return np.where(m > 0, c, F32(1.0)).astype(F32)


def quantize_rowwise(X_f16: np.ndarray, idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Step 2 split + Step 4 row quantisation of X.

    [DIGEST] "The Full LLM.int8() Algorithm", Step 2 (split X into X^O and
    X^{not O}) and Step 4, first and third bullets: c_x_i is 127 over the
    absmax of row i of X^{not O}; X_i8 = round(c_x ⊙ X^{not O}).
    [TM] "The mixed-precision decomposition" (the regular term holds no
    outliers, so its per-row absmax is small).

    Returns Xq int8 [s, h] with the O columns set to 0 (so a full-width integer
    product equals the sum over the non-outlier columns), c_x fp32 [s], and
    X_O fp16 [s, |O|] = the outlier columns in ascending order of index.
    """
    X16 = np.asarray(X_f16, dtype=np.float16)
    s, h = X16.shape
    idx = np.asarray(idx, dtype=np.int64)
    regular = np.ones(h, dtype=bool)
    regular[idx] = False
    X32 = X16.astype(F32)
    if regular.any() and s > 0:
        m = np.abs(X32[:, regular]).max(axis=1)
    else:
        m = np.zeros(s, dtype=F32)
    c_x = row_scales(m)
    v = (X32 * c_x[:, None]).astype(F32)            # one fp32 multiply
    q = np.clip(round_half_away(v), -127, 127)
    q[:, ~regular] = 0
    Xq = q.astype(np.int8)
    X_O = X16[:, idx].copy()
    return Xq, c_x, X_O


def quantize_colwise_weights(W_f16: np.ndarray, col_chunk: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """Load-time conversion W -> (Wq_t int8 [o, h] = W_i8 transposed, c_w fp32 [o]).

    [DIGEST] "The Full LLM.int8() Algorithm", Step 4 second and third bullets:
    c_w_j = 127 / max_i |W_ij|, W_i8 = round(W ⊙ c_w); [DIGEST] "Why
    vector-wise rather than row-wise" (column constants are precomputed once
    at load time). Reading: because the constants are fixed at load time while
    O changes every forward, the max runs over all h rows of W (parity
    unpinned: a convention, not a page fact). Columns are independent, so
    they are processed in chunks to bound memory; this changes no arithmetic.
    """
    W16 = np.asarray(W_f16, dtype=np.float16)
    h, o = W16.shape
    Wq_t = np.empty((o, h), dtype=np.int8)
    c_w = np.empty(o, dtype=F32)
    for j0 in range(0, o, col_chunk):
        j1 = min(o, j0 + col_chunk)
        W32 = W16[:, j0:j1].astype(F32)
        m = np.abs(W32).max(axis=0) if h > 0 else np.zeros(j1 - j0, dtype=F32)
        c = row_scales(m)
        v = (W32 * c[None, :]).astype(F32)
        q = np.clip(round_half_away(v), -127, 127).astype(np.int8)
        Wq_t[j0:j1] = q.T
        c_w[j0:j1] = c
    return Wq_t, c_w


def int8_matmul_i32(Xq: np.ndarray, Wq_t: np.ndarray, col_chunk: int = 4096) -> np.ndarray:
    """Step 4, fourth bullet: C_i32 = X_i8 x W_i8, exact.

    [DIGEST] "The Full LLM.int8() Algorithm", Step 4 (Int8 matrix
    multiplication producing an Int32 accumulator). Computed as a float64
    product of int8-valued arrays (exact: see the module docstring), in
    output-column chunks to bound memory.
    """
    s, h = Xq.shape
    o = Wq_t.shape[0]
    out = np.empty((s, o), dtype=np.int32)
    A = Xq.astype(F64)
    for j0 in range(0, o, col_chunk):
        j1 = min(o, j0 + col_chunk)
        B = Wq_t[j0:j1].astype(F64)
        out[:, j0:j1] = (A @ B.T).astype(np.int64).astype(np.int32)
    return out


def outlier_matmul(X_O: np.ndarray, W_f16: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Step 3: C^O = X^O_f16 x W^O_f16 in float64 (products of fp16 are exact).

    [DIGEST] "The Full LLM.int8() Algorithm", Step 3; [TM] "The
    mixed-precision decomposition" (sum over k in O of X[:,k] W[k,:]);
    [PY] "第二件武器：混合精度分解" (W row h follows X column h).
    W^O are the rows of the original fp16 W indexed by O.
    """
    idx = np.asarray(idx, dtype=np.int64)
    W16 = np.asarray(W_f16, dtype=np.float16)
    A = np.asarray(X_O, dtype=np.float16).astype(F64)
    B = W16[idx, :].astype(F64)
    return A @ B


def dequantize_and_add(C_i32: np.ndarray, c_x: np.ndarray, c_w: np.ndarray,
                       C_O: Optional[np.ndarray], bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Step 4 last bullet and Step 5: C = S ⊙ C_i32 + C^O, S_ij = 1/(c_x_i c_w_j).

    [DIGEST] "The Full LLM.int8() Algorithm", Step 4 (dequantise with the
    outer product of the scales) and Step 5 (sum the two partial results);
    [PY] "第一件武器：向量级量化" (divide by c_x ⊗ c_w). Evaluated in float64
    and rounded once to fp16.

    bias (fp16 [o], optional) is the linear layer's bias, which stays in
    16 bit ([DIGEST] "Mixed-Precision Decomposition", memory accounting):
    b_j is added to every row of column j in the same float64 sum, before
    the single rounding.
    """
    denom = c_x.astype(F64)[:, None] * c_w.astype(F64)[None, :]   # exact
    C = C_i32.astype(F64) / denom
    if C_O is not None:
        C = C + C_O
    if bias is not None:
        C = C + np.asarray(bias, dtype=np.float16).astype(F64)[None, :]
    return C.astype(np.float16)


def dequantized_outlier_rows(Wq_t: np.ndarray, c_w: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Outlier rows W^O when no fp16 copy of W is kept (a storage variant; the
    pages' Step 3 uses the original fp16 rows, [DIGEST] "The Full LLM.int8()
    Algorithm"): the int8 code dequantised by multiplying back with the
    inverse scale ([PY] "量化为什么会崩：一个尺度统治全局":
    dequantisation multiplies back by 1/s), W^O[k, j] = fl16(fl32(W_i8[idx[k], j]
    * fl32(1 / c_w[j]))): the reciprocal and the product each rounded to
    fp32, the result rounded once to fp16. Only the int8 weights and their
    scales then stay resident, the memory saving of [DIGEST] "Executive
    Summary" (1.96x on BLOOM-176B)."""
    idx = np.asarray(idx, dtype=np.int64)
    q = Wq_t[:, idx].T.astype(F32)                        # [|O|, o], exact
    inv = (F32(1.0) / np.asarray(c_w, dtype=F32)).astype(F32)
    return (q * inv[None, :]).astype(F32).astype(np.float16)


def int8_mixed_matmul(Xq: np.ndarray, c_x: np.ndarray, X_O: np.ndarray, idx: np.ndarray,
                      Wq_t: np.ndarray, c_w: np.ndarray, W_f16: Optional[np.ndarray],
                      col_chunk: int = 4096, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Steps 3-5 given the quantised operands: C fp16 [s, o]. With W_f16 None
    the outlier rows come from dequantized_outlier_rows (no resident fp16 W);
    bias (fp16 [o]) is added as in dequantize_and_add."""
    s = Xq.shape[0]
    o = Wq_t.shape[0]
    C = np.empty((s, o), dtype=np.float16)
    for j0 in range(0, o, col_chunk):
        j1 = min(o, j0 + col_chunk)
        Ci = int8_matmul_i32(Xq, Wq_t[j0:j1], col_chunk=col_chunk)
        if W_f16 is None:
            rows = dequantized_outlier_rows(Wq_t[j0:j1], c_w[j0:j1], idx).astype(F64)
            CO = np.asarray(X_O, dtype=np.float16).astype(F64) @ rows
        else:
            CO = outlier_matmul(X_O, W_f16[:, j0:j1], idx)
        C[:, j0:j1] = dequantize_and_add(Ci, c_x, c_w[j0:j1], CO, None if bias is None else bias[j0:j1])
    return C


def fp16_matmul(X_f16: np.ndarray, W_f16: np.ndarray, col_chunk: int = 4096) -> np.ndarray:
    """The FP16 baseline of [DIGEST] "Runtime Performance (Appendix D)"
    (Table 5 reports every variant as a speed-up over the FP16 matrix
    multiply of the same layer): C = fp16(X W), the product taken in float64
    and rounded once to fp16 (round to nearest even).

    Each float64 product of two fp16 values is exact; the sum over h is
    rounded in float64, far below one fp16 ulp of the result.
    """
    Xd = X_f16.astype(np.float64)
    o = W_f16.shape[1]
    C = np.empty((X_f16.shape[0], o), np.float16)
    for j0 in range(0, o, col_chunk):
        C[:, j0:j0 + col_chunk] = (Xd @ W_f16[:, j0:j0 + col_chunk].astype(np.float64)).astype(np.float16)
    return C


def forward(X_f16: np.ndarray, W_f16: np.ndarray, alpha: float = 6.0,
            Wq_t: Optional[np.ndarray] = None, c_w: Optional[np.ndarray] = None,
            keep: bool = False, fp16_weights: bool = True,
            bias: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole procedure for one linear layer ([DIGEST] Steps 1-5 in order).

    If (Wq_t, c_w) are given they are the load-time conversion of W_f16;
    otherwise it is done here. With fp16_weights False the outlier product
    uses dequantized_outlier_rows instead of the fp16 rows of W_f16 (the
    storage variant without a resident fp16 W). bias (fp16 [o], optional) is
    the layer's bias, added before the single rounding of C. Returns a dict
    with C and the intermediates.
    """
    mask, idx, n_out = outlier_columns(X_f16, alpha)                 # Step 1
    Xq, c_x, X_O = quantize_rowwise(X_f16, idx)                       # Steps 2, 4
    if Wq_t is None or c_w is None:
        Wq_t, c_w = quantize_colwise_weights(W_f16)                   # Step 4 (load time)
    C = int8_mixed_matmul(Xq, c_x, X_O, idx, Wq_t, c_w, W_f16 if fp16_weights else None,
                          bias=bias)                                   # Steps 3, 4, 5
    out = {"C": C, "mask": mask, "idx": idx, "n_out": np.int32(n_out),
           "Xq": Xq, "c_x": c_x, "X_O": X_O}
    if keep:
        out["Wq_t"] = Wq_t
        out["c_w"] = c_w
    return out
