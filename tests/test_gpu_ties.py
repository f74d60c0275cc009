"""Exact rounding ties and the alpha near miss through every GPU quantiser
launch shape, compared bit for bit with the oracle.

Under fp32 scales some products land exactly on a half: with the absmax
m = 1.1162109375 (fp16), x = +-0.00439453125 gives fl32(x fl32(127 / m)) =
+-0.5 and x = +-0.02197265625 gives +-2.5. Rounding to nearest ([TM]
"Absmax INT8 quantization from first principles") with ties away from zero
maps them to +-1 and +-3; ties to even would give 0 and +-2. The inputs
below hold such ties in almost every element, at every chunk position of
every wavefront part, so each launch shape of each quantiser rounds
thousands of them. Each row (column) also holds +m and -m, so its zero
point is 0 and the zeropoint codes are the absmax codes, ties included.
A column whose only large value is 5.99609375 (the fp16 value just below
alpha = 6) must stay out of O ([DIGEST] "The Full LLM.int8() Algorithm",
Step 1), and two columns holding 10.0 / -12.0 in one row are in O and are
excluded from the row constants (Step 4).
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
import oracle.variants as ov
from gpu_util import DEV, H, T, check_detect, check_rows, say

pytestmark = pytest.mark.gpu

M = 1.1162109375
TIES = np.array([0.00439453125, -0.00439453125, 0.02197265625, -0.02197265625], np.float16)
NEAR_MISS_COL = 9


def tie_matrix(rows: int, cols: int, outliers: bool = True, near_miss: bool = True) -> np.ndarray:
    """[rows, cols] fp16: ties everywhere, +m and -m in every row, optional
    outlier columns (5 and cols - 3) and near-miss column (9)."""
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    X = TIES[(r + c) % 4].copy()
    ocols = [5, cols - 3] if outliers else []
    skip = set(ocols) | ({NEAR_MISS_COL} if near_miss else set())
    for i in range(rows):
        pos, neg = (7 * i) % cols, (7 * i + 3) % cols
        pos = pos + 1 if pos in skip else pos
        neg = neg + 1 if neg in skip else neg
        X[i, pos] = M
        X[i, neg] = -M
    for oc in ocols:
        X[0, oc] = 10.0
        X[rows - 1, oc] = -12.0
    if near_miss:
        X[1 % rows, NEAR_MISS_COL] = 5.99609375
    return X


def _tie_fraction(X: np.ndarray, c: np.ndarray, axis_rows: bool = True) -> float:
    """Fraction of the products x * c that are exact halves."""
    c = np.asarray(c, np.float32)
    v = (X.astype(np.float32) * (c[:, None] if axis_rows else c[None, :])).astype(np.float32)
    return float((np.abs(v.astype(np.float64)) % 1.0 == 0.5).mean())


def _check_tie_codes(X: np.ndarray, Xq_r: np.ndarray, c_r: np.ndarray, idx_r: np.ndarray) -> None:
    """The input really exercises the ties: in the rows whose constant is
    fl32(127 / m), each tie value carries the code rounded away from zero."""
    rows = np.asarray(c_r, np.float32) == np.float32(127.0) / np.float32(M)
    reg = np.ones(X.shape[1], bool)
    reg[idx_r] = False
    for x, q in zip(TIES, (1, -1, 3, -3)):
        sel = (X == x) & rows[:, None] & reg[None, :]
        assert sel.any() and (Xq_r[sel] == q).all()


def _detect(X):
    mask, idx, n_out = i8.detect_outlier_cols(T(X), 6.0)
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, mask, idx, n_out)
    return mask, idx, n_out, idx_r


# (s, h): every launch shape of the absmax row quantiser k_quant_rows, named
# by the wavefronts per row (W) and 16-byte chunks per lane (CPL; 0 = the
# row re-read instead of held in registers) that the launch picks.
ROW_SHAPES = [(64, 256, "W4 CPL2"), (64, 8192, "W4 CPL4"), (16, 16384, "W4 CPL8"), (4, 32768, "W4 CPL16"),
              (8, 65536, "W1 CPL0"),
              (2048, 1024, "W2 CPL2"), (2048, 4096, "W2 CPL4"), (2048, 8192, "W2 CPL8"), (4096, 8192, "W2 CPL8 many"),
              (4096, 512, "W1 CPL2"), (4096, 2048, "W1 CPL4"), (4096, 4096, "W1 CPL8"),
              (4096, 12288, "W4 CPL8 many"), (4096, 8256, "W4 CPL8 ragged")]


@pytest.mark.parametrize("s,h,label", ROW_SHAPES, ids=[c[2] for c in ROW_SHAPES])
def test_row_quantiser_ties(s, h, label):
    X = tie_matrix(s, h)
    say(f"  launch: detect + quantize_rowwise {label} s={s} h={h}")
    mask, idx, n_out, idx_r = _detect(X)
    assert idx_r.tolist() == [5, h - 3]
    Xq, c_x, X_O = i8.quantize_rowwise(T(X), mask, idx, n_out)
    torch.cuda.synchronize()
    Xq_r, cx_r, _ = check_rows(X, idx_r, Xq, c_x, X_O)
    assert _tie_fraction(X, cx_r) > 0.5
    _check_tie_codes(X, Xq_r, cx_r, idx_r)
    assert Xq_r[1 % s, NEAR_MISS_COL] == 127     # the near miss sets its row's constant


# (s, h): the few-row forward (s <= 8: in one launch up to 24 KiB of X,
# else detection and row quantisation by slabs of 128 columns in one row
# group of 16) and detection + row pass beside each product: the K-split
# (s <= 16) and column-split (s <= 128) weight streams and the tiled product.
FORWARD_SHAPES = [(8, 256, "one launch"), (8, 2048, "slabs"), (8, 12288, "slabs wide"), (16, 12288, "rows K-split"),
                  (24, 1024, "rows column-split"), (48, 4096, "rows column-split 3"),
                  (64, 12288, "rows column-split 4 wide"), (300, 2048, "rows tiled")]


@pytest.mark.parametrize("s,h,label", FORWARD_SHAPES, ids=[c[2] for c in FORWARD_SHAPES])
def test_forward_prologue_ties(s, h, label):
    o = 128
    X = tie_matrix(s, h)
    rng = np.random.default_rng(s + h)
    W = (0.02 * rng.standard_normal((h, o), dtype=np.float32)).astype(np.float16)
    say(f"  launch: forward {label} s={s} h={h} o={o}")
    Wd = T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(T(X), Wq, c_w, Wd, 6.0, workspace=ws)
    torch.cuda.synchronize()
    v = i8.forward_workspace_views(ws, s, h)
    idx_r = check_detect(X, 6.0, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == [5, h - 3]
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    assert _tie_fraction(X, cx_r) > 0.5
    _check_tie_codes(X, Xq_r, cx_r, idx_r)
    assert not H(v["acc"]).any(), "forward left its accumulator non-zero"
    ref = oracle.forward(X, W, 6.0)
    R = ref["C"].astype(np.float64)
    assert np.abs(H(C).astype(np.float64) - R).max() <= 2e-3 * np.abs(R).max()


# (s, h): launch shapes of the tensor-wise row passes and of the zeropoint
# row quantiser (the same lists as their parity tests).
TW_ROW_SHAPES = [(8, 1024, "W4 CPL2"), (64, 8192, "W4 CPL4"), (16, 16384, "W4 CPL8"), (4, 32768, "W4 CPL16"),
                 (3, 40960, "one wavefront per row"), (2048, 256, "many rows")]
ZP_ROW_SHAPES = [(2048, 256, "W2 CPL2"), (2048, 4096, "W2 CPL4"), (2048, 8192, "W2 CPL8"),
                 (4096, 256, "W1 CPL2"), (4096, 2048, "W1 CPL4"), (64, 8192, "W4 CPL4"),
                 (16, 16384, "W4 CPL8"), (4, 32768, "W4 CPL16"), (3, 40960, "two-pass")]


@pytest.mark.parametrize("s,h,label", TW_ROW_SHAPES, ids=[c[2] for c in TW_ROW_SHAPES])
def test_tensorwise_row_ties(s, h, label):
    X = tie_matrix(s, h, near_miss=False)     # one constant over all rows: m is the tensor's absmax
    say(f"  launch: tensor-wise rows {label} s={s} h={h}")
    mask, idx, n_out, idx_r = _detect(X)
    Xq, c_x, X_O = i8.quantize_tensorwise(T(X), mask, idx, n_out)
    torch.cuda.synchronize()
    Xq_r, cx_r, _ = ov.quantize_tensorwise(X, idx_r)
    assert _tie_fraction(X, cx_r) > 0.5
    assert np.array_equal(H(Xq), Xq_r), "tensor-wise Xq differs"
    assert np.array_equal(H(c_x).view(np.uint32), cx_r.view(np.uint32)), "tensor-wise c_x differs"


@pytest.mark.parametrize("s,h,label", ZP_ROW_SHAPES, ids=[c[2] for c in ZP_ROW_SHAPES])
def test_zeropoint_row_ties(s, h, label):
    X = tie_matrix(s, h)
    say(f"  launch: zeropoint rows {label} s={s} h={h}")
    mask, idx, n_out, idx_r = _detect(X)
    Xq, nd_x, zp_x, rs_x, X_O = i8.quantize_rowwise_zeropoint(T(X), mask, idx, n_out)
    torch.cuda.synchronize()
    Xq_r, ndx_r, zpx_r, _ = ov.quantize_rowwise_zeropoint(X, idx_r)
    assert _tie_fraction(X, ndx_r) > 0.5
    assert (zpx_r[2:] == 0).all()
    assert np.array_equal(H(Xq), Xq_r), "zeropoint Xq differs"
    assert np.array_equal(H(nd_x).view(np.uint32), ndx_r.view(np.uint32)), "nd_x differs"
    assert np.array_equal(H(zp_x), zpx_r), "zp_x differs"
    assert np.array_equal(H(rs_x), Xq_r.astype(np.int64).sum(axis=1)), "rowsum_x differs"


WEIGHT_SHAPES = [(256, 128), (4096, 192), (12288, 64)]


@pytest.mark.parametrize("h,o", WEIGHT_SHAPES)
def test_weight_conversion_ties(h, o):
    """Columns of W holding the tie pattern, +m and -m: the absmax (vector),
    tensor-wise and zeropoint conversions, codes and constants bit for bit."""
    W = np.ascontiguousarray(tie_matrix(o, h, outliers=False, near_miss=False).T)   # column j = row j above
    Wd = T(W)
    say(f"  launch: weight conversions h={h} o={o}")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    Wt, c_t = i8.quantize_weights_tensorwise(Wd)
    Wz, nd_w, zp_w, cs_w = i8.quantize_colwise_weights_zeropoint(Wd)
    torch.cuda.synchronize()
    Wq_r, cw_r = oracle.quantize_colwise_weights(W)
    assert _tie_fraction(W, cw_r, axis_rows=False) > 0.9
    assert np.array_equal(H(i8.panels_to_rows(Wq)), Wq_r), "Wq differs"
    assert np.array_equal(H(c_w).view(np.uint32), cw_r.view(np.uint32)), "c_w differs"
    Wt_r, ct_r = ov.quantize_weights_tensorwise(W)
    assert np.array_equal(H(i8.panels_to_rows(Wt)), Wt_r), "tensor-wise Wq differs"
    assert np.array_equal(H(c_t).view(np.uint32), ct_r.view(np.uint32)), "tensor-wise c_w differs"
    Wz_r, ndw_r, zpw_r = ov.quantize_colwise_weights_zeropoint(W)
    assert (zpw_r == 0).all()
    assert np.array_equal(H(i8.panels_to_rows(Wz)), Wz_r), "zeropoint Wq differs"
    assert np.array_equal(H(nd_w).view(np.uint32), ndw_r.view(np.uint32)), "nd_w differs"
    assert np.array_equal(H(zp_w), zpw_r), "zp_w differs"
    assert np.array_equal(H(cs_w), Wz_r.astype(np.int64).sum(axis=1)), "colsum_w differs"


@pytest.mark.parametrize("s,h,path", [(4, 256, "detect"), (100, 256, "detect"), (8, 256, "forward, one launch"),
                                      (8, 2048, "forward, slab pair"), (100, 256, "forward, many rows")])
def test_detection_with_nan(s, h, path):
    """A column is in O when one of its elements reaches alpha ([DIGEST] "The
    Full LLM.int8() Algorithm", Step 1), also when it holds a NaN as well;
    a NaN alone does not reach alpha. Only the outlier set is defined for
    such inputs, so only the mask, the index list and |O| are compared."""
    X = tie_matrix(s, h, outliers=False, near_miss=False)
    X[0, 3] = np.nan
    X[s - 1, 3] = 10.0                 # NaN and an outlier: in O
    X[1, 7] = np.nan                   # NaN only: not in O
    X[0, 20] = -np.nan
    X[2, 20] = 5.99609375              # NaN and a near miss: not in O
    X[3, 33] = -6.0                    # plain outlier: in O
    X[:, 200] = np.nan
    X[s - 1, 200] = 6.0                # NaN in every other row and alpha: in O
    X[s // 2, h - 1] = np.nan          # NaN only, last column
    say(f"  launch: {path} with NaN s={s} h={h}")
    if path == "detect":
        mask, idx, n_out = i8.detect_outlier_cols(T(X), 6.0)
    else:
        o = 64
        W = np.zeros((h, o), np.float16)
        Wd = T(W)
        Wq, c_w = i8.quantize_colwise_weights(Wd)
        ws = i8.forward_workspace(s, h, DEV)
        i8.forward(T(X), Wq, c_w, Wd, 6.0, workspace=ws)
        v = i8.forward_workspace_views(ws, s, h)
        mask, idx, n_out = v["mask"], v["idx"], v["n_out"]
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, mask, idx, n_out)
    assert idx_r.tolist() == [3, 33, 200]
