"""Pins of the oracle's quantiser variants (oracle/variants.py) to facts the
pages and mathematics fix: the pages' tensor-wise illustration, reductions
to the main path where the constants coincide, the zeropoint map's range
and round-trip bound, the pages' four-term product identity, an exact
rational brute force, and a closed-form error bound that a dropped zero
point violates.

Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
Transformers at Scale" (paper-graph-ui digest); [PY] "LLM.int8() 完全拆解"
(pinghaoyang.com.cn).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import rational
from workloads import random_case

INF = float("inf")


def _symmetrise_rows(X, idx):
    """Set two regular columns of every row to +m and -m, m the row's absmax
    over the regular columns, so each row's regular min is -max."""
    X = X.copy()
    h = X.shape[1]
    reg = np.setdiff1d(np.arange(h), idx)
    a, b = reg[0], reg[1]
    m = np.abs(X[:, reg].astype(np.float32)).max(axis=1)
    X[:, a] = m.astype(np.float16)
    X[:, b] = (-m).astype(np.float16)
    return X


def _symmetrise_cols(W):
    W = W.copy()
    m = np.abs(W.astype(np.float32)).max(axis=0)
    W[0, :] = m.astype(np.float16)
    W[1, :] = (-m).astype(np.float16)
    return W


# ---------------------------------------------------------------- tensor-wise and row-wise

def test_tensorwise_illustration():
    """[DIGEST] "Quantization Primitives": with one value 60 in the tensor,
    values in [-3, 3] map into [-6.35, 6.35]; under one constant per tensor
    that holds for a row that has no outlier of its own, while row-wise
    quantisation gives that row the full range."""
    X = np.zeros((2, 64), np.float16)
    X[0, 5] = 60.0
    X[1, :4] = [3.0, -3.0, 1.5, -0.75]
    Xq, c_x, _ = oracle.quantize_tensorwise(X, np.zeros(0, np.int64))
    assert (c_x == np.float32(127.0) / np.float32(60.0)).all()
    assert Xq[1, :4].tolist() == [6, -6, 3, -2]         # 6.35, 3.175, 1.59 rounded
    assert abs(3.0 * float(c_x[1]) - 6.35) < 1e-2
    Xr, c_r, _ = oracle.quantize_rowwise(X, np.zeros(0, np.int64))
    assert Xr[1, :2].tolist() == [127, -127]


def test_tensorwise_weights_one_constant():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((96, 40)) * 0.02).astype(np.float16)
    Wq_t, c_w = oracle.quantize_weights_tensorwise(W)
    m = np.abs(W.astype(np.float32)).max()
    assert (c_w == np.float32(127.0) / m).all()
    j, k = np.unravel_index(np.argmax(np.abs(W.astype(np.float32))), W.shape)
    assert abs(int(Wq_t[k, j])) == 127
    assert np.abs(Wq_t.astype(np.int32)).max() == 127


def test_schemes_agree_when_constants_coincide():
    """Every row of X with the same absmax and every column of W with the
    same absmax: tensor-wise, row-wise and vector-wise quantisation use the
    same constants and give the same C bit for bit (with and without the
    decomposition)."""
    for alpha, nout in ((6.0, 3), (INF, 0)):
        inp = random_case(7, 12, 256, 96, nout, row_frac=0.5)
        X, W = inp["X"].copy(), inp["W"].copy()
        # regular values stay below 5.5 (the generator redraws larger ones)
        X[:, 10] = np.float16(5.5) * np.where(np.arange(12) % 2, 1, -1).astype(np.float16)
        W[20, :] = np.float16(0.125)
        t = oracle.variant_forward(X, W, "tensor", alpha)
        r = oracle.variant_forward(X, W, "row", alpha)
        v = oracle.variant_forward(X, W, "vector", alpha)
        assert np.array_equal(t.view(np.uint16), v.view(np.uint16))
        assert np.array_equal(r.view(np.uint16), v.view(np.uint16))


def test_rowwise_equals_vectorwise_only_when_weight_columns_agree():
    """Row-wise (row constants for X, one constant for W, [DIGEST]
    "Vector-wise Quantization") equals vector-wise when every column of W has
    the same absmax; with columns of different absmax it does not."""
    inp = random_case(8, 10, 192, 64, 2, row_frac=0.5)
    X, W = inp["X"], inp["W"].copy()
    W[5, :] = np.float16(0.1)
    r = oracle.variant_forward(X, W, "row")
    v = oracle.variant_forward(X, W, "vector")
    assert np.array_equal(r.view(np.uint16), v.view(np.uint16))
    W2 = inp["W"]
    assert not np.array_equal(oracle.variant_forward(X, W2, "row"), oracle.variant_forward(X, W2, "vector"))


# ---------------------------------------------------------------- zeropoint

def test_zeropoint_one_sided_data_uses_the_whole_range():
    """[DIGEST] "Quantization Primitives" / [PY]: for one-signed data (a ReLU
    output) the zeropoint map sends min to -127 and max to 127 (all 255
    codes available), where absmax uses only [0, 127]."""
    rng = np.random.default_rng(5)
    X = np.abs(rng.standard_normal((6, 128))).astype(np.float16)
    Xq, nd, zp, _ = oracle.quantize_rowwise_zeropoint(X, np.zeros(0, np.int64))
    for i in range(6):
        assert Xq[i, np.argmin(X[i])] == -127 and Xq[i, np.argmax(X[i])] == 127
    Xa, _, _ = oracle.quantize_rowwise(X, np.zeros(0, np.int64))
    assert Xa.min() >= 0
    assert len(np.unique(Xq)) > 1.5 * len(np.unique(Xa))


def test_zeropoint_symmetric_data_reduces_to_absmax():
    """Rows and columns whose min is -max: nd = 254 / (2 max) = 127 / max
    is the absmax constant and zp = 0, so the codes and C equal the
    vector-wise absmax path's bit for bit."""
    inp = random_case(9, 10, 192, 48, 2, row_frac=0.5)
    for alpha in (6.0, INF):
        _, idx, _ = oracle.outlier_columns(inp["X"], alpha)
        X = _symmetrise_rows(inp["X"], idx)
        W = _symmetrise_cols(inp["W"])
        Xq, nd, zp, _ = oracle.quantize_rowwise_zeropoint(X, idx)
        Xa, c_x, _ = oracle.quantize_rowwise(X, idx)
        assert not zp.any() and np.array_equal(nd, c_x) and np.array_equal(Xq, Xa)
        Wq_t, nd_w, zp_w = oracle.quantize_colwise_weights_zeropoint(W)
        Wa_t, c_w = oracle.quantize_colwise_weights(W)
        assert not zp_w.any() and np.array_equal(nd_w, c_w) and np.array_equal(Wq_t, Wa_t)
        z = oracle.variant_forward(X, W, "zeropoint", alpha)
        v = oracle.variant_forward(X, W, "vector", alpha)
        assert np.array_equal(z.view(np.uint16), v.view(np.uint16))


def test_zeropoint_roundtrip_bound():
    """(q + zp) / nd reconstructs x within half a step (plus the fp32
    rounding of nd x); a code clamped at +-127 is within 1.5 steps."""
    rng = np.random.default_rng(6)
    X = (rng.standard_normal((40, 256)) * rng.uniform(0.1, 10, (40, 1)) + rng.uniform(-5, 5, (40, 1)))
    X = X.astype(np.float16)
    Xq, nd, zp, _ = oracle.quantize_rowwise_zeropoint(X, np.zeros(0, np.int64))
    x = X.astype(np.float64)
    rec = (Xq.astype(np.float64) + zp[:, None]) / nd.astype(np.float64)[:, None]
    err = np.abs(rec - x)
    step = 1.0 / nd.astype(np.float64)[:, None]
    unclamped = np.abs(Xq) < 127
    assert (err[unclamped] <= (0.5 * step + np.abs(x) * 2.0 ** -23)[unclamped]).all()
    assert (err <= 1.5 * step + np.abs(x) * 2.0 ** -23).all()


def test_four_term_expansion_identity():
    """The pages' expansion ([DIGEST] "Quantization Primitives"; [PY]
    "量化为什么会崩：一个尺度统治全局"): (A + zp_a)(B + zp_b) = AB + A zp_b + zp_a B + zp_a zp_b,
    summed over the non-outlier columns, evaluated term by term with Python
    integers, equals the oracle's product of the shifted codes."""
    inp = random_case(11, 5, 64, 9, 2, row_frac=0.6)
    X, W = inp["X"], inp["W"]
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    Xq, nd_x, zp_x, _ = oracle.quantize_rowwise_zeropoint(X, idx)
    Wq_t, nd_w, zp_w = oracle.quantize_colwise_weights_zeropoint(W)
    Cp = oracle.zeropoint_product_i64(Xq, zp_x, Wq_t, zp_w, idx)
    reg = [k for k in range(64) if k not in set(idx.tolist())]
    for i in range(5):
        for j in range(9):
            za, zb = int(zp_x[i]), int(zp_w[j])
            ab = sum(int(Xq[i, k]) * int(Wq_t[j, k]) for k in reg)
            a_sum = sum(int(Xq[i, k]) for k in reg)
            b_sum = sum(int(Wq_t[j, k]) for k in reg)
            assert int(Cp[i, j]) == ab + a_sum * zb + za * b_sum + len(reg) * za * zb


@pytest.mark.parametrize("seed,s,h,o,nout", [(20, 4, 32, 6, 1), (21, 5, 64, 8, 0), (22, 3, 96, 5, 3)])
def test_zeropoint_exact_rational_bruteforce(seed, s, h, o, nout):
    """Exact rational evaluation (IEEE rounding emulated from its definition)
    agrees with the oracle: nd, zp and the codes exactly, C' exactly, C
    within one fp16 ulp (almost always equal)."""
    inp = random_case(seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    X[1] = np.abs(X[1])                                      # a one-signed row
    O, nd_x, zp_x, Xq, nd_w, zp_w, Wq, Cp, C = rational.zeropoint_brute_force(X, W, 6.0)
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    assert idx.tolist() == O
    oXq, ond_x, ozp_x, oXO = oracle.quantize_rowwise_zeropoint(X, idx)
    oWq_t, ond_w, ozp_w = oracle.quantize_colwise_weights_zeropoint(W)
    assert [Fraction(float(v)) for v in ond_x] == nd_x and ozp_x.tolist() == zp_x
    assert [Fraction(float(v)) for v in ond_w] == nd_w and ozp_w.tolist() == zp_w
    assert oXq.tolist() == Xq and oWq_t.T.tolist() == Wq
    assert oracle.zeropoint_product_i64(oXq, ozp_x, oWq_t, ozp_w, idx).tolist() == Cp
    oC = oracle.zeropoint_matmul(oXq, ond_x, ozp_x, oXO, idx, oWq_t, ond_w, ozp_w, W)
    equal = 0
    for i in range(s):
        for j in range(o):
            g = Fraction(float(oC[i, j]))
            assert abs(g - C[i][j]) <= rational.ulp16(C[i][j])
            equal += g == C[i][j]
    assert equal >= s * o - 1


def _zp_error_bound(X, W, idx, nd_x, nd_w):
    """|C - X W| <= sum over regular k of (ex |w| + |x| ew + ex ew) + half an
    fp16 ulp, with ex = 1.5 / nd_x + |x| 2^-23 (likewise ew): the round-trip
    bound above carried through the product."""
    h = X.shape[1]
    reg = np.setdiff1d(np.arange(h), idx)
    x = np.abs(X[:, reg].astype(np.float64))
    w = np.abs(W[reg].astype(np.float64))
    ex = 1.5 / nd_x.astype(np.float64)[:, None] + x * 2.0 ** -23
    ew = 1.5 / nd_w.astype(np.float64)[None, :] + w * 2.0 ** -23
    return ex @ w + x @ ew + ex @ ew


def test_zeropoint_closed_form_error_bound_and_planted_mistake():
    """C of the zeropoint path is within the closed-form bound of the exact
    X W; the same codes with the zero points dropped (q / nd in place of
    (q + zp) / nd) are not."""
    inp = random_case(12, 16, 256, 64, 3, row_frac=0.5)
    X, W = inp["X"].copy(), inp["W"]
    X[:8] = np.abs(X[:8])                                    # one-signed rows: zp far from 0
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    Xq, nd_x, zp_x, X_O = oracle.quantize_rowwise_zeropoint(X, idx)
    Wq_t, nd_w, zp_w = oracle.quantize_colwise_weights_zeropoint(W)
    C = oracle.zeropoint_matmul(Xq, nd_x, zp_x, X_O, idx, Wq_t, nd_w, zp_w, W).astype(np.float64)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    bound = _zp_error_bound(X, W, idx, nd_x, nd_w)
    half_ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert (np.abs(C - exact) <= bound + half_ulp).all()
    wrong = oracle.zeropoint_matmul(Xq, nd_x, np.zeros_like(zp_x), X_O, idx, Wq_t, nd_w, zp_w, W)
    assert (np.abs(wrong.astype(np.float64) - exact) > bound + half_ulp).any()


def test_zeropoint_constant_row_convention():
    """Convention (parity unpinned: the pages are silent): a row whose
    regular values are all equal gets nd = 1; an all-zero row is exact."""
    X = np.zeros((2, 64), np.float16)
    X[1, :] = 2.0
    Xq, nd, zp, _ = oracle.quantize_rowwise_zeropoint(X, np.zeros(0, np.int64))
    assert (nd == 1).all()
    assert ((Xq[0].astype(int) + zp[0]) == 0).all()
    assert ((Xq[1].astype(int) + zp[1]) == 2).all()
