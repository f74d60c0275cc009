"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the
pages print for worked examples (tests/golden/worked_examples.json), closed
forms, invariants, special cases that reduce to a textbook routine, and an
exact rational brute force (tests/rational.py) on tiny inputs.

Page tags: [TM] transformer-math LLM.int8() tutorial (aicassindra.com);
[DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale"
(paper-graph-ui digest); [PY] "LLM.int8() 完全拆解" (pinghaoyang.com.cn).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import rational
from workloads import get_config, make_inputs, random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
INF = float("inf")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _alpha(a):
    return INF if a == "inf" else float(a)


def _ulp16(x):
    x = np.abs(np.asarray(x, dtype=np.float16))
    return (np.spacing(x.astype(np.float16)).astype(np.float64))


# ---------------------------------------------------------------- printed values

@pytest.mark.parametrize("case", _golden()["rows"], ids=lambda c: c["name"])
def test_worked_rows(case):
    """[TM] 'A worked quantization example', 'Why one outlier crushes a whole
    vector' and the decomposition applied to the latter."""
    x = np.array([case["x"]], dtype=np.float16)
    mask, idx, n = oracle.outlier_columns(x, _alpha(case["alpha"]))
    assert list(idx) == case.get("O", [])
    Xq, c_x, X_O = oracle.quantize_rowwise(x, idx)
    assert Xq[0].tolist() == case["Q"]
    assert float(np.abs(x.astype(np.float32)[0][~np.isin(np.arange(4), idx)]).max()) == case["absmax"]
    if "scale_printed" in case:
        assert round(float(c_x[0]), case["scale_decimals"]) == pytest.approx(case["scale_printed"])
    if "xhat_printed" in case:
        xhat = Xq[0].astype(np.float64) / float(c_x[0])
        d = case["xhat_decimals"]
        np.testing.assert_allclose(np.round(xhat, d), case["xhat_printed"], atol=0.6 * 10 ** -d)
    if "roundtrip_err_printed" in case:
        xhat = Xq[0].astype(np.float64) / float(c_x[0])
        assert np.abs(xhat - x[0].astype(np.float64)).max() <= case["roundtrip_err_printed"]
    if "X_O" in case:
        assert X_O[0].astype(np.float64).tolist() == case["X_O"]
        assert n == len(case["O"])
        assert mask[0] == sum(1 << j for j in case["O"])


def test_worked_row_fp32_scale_exact():
    """With fp32 scales the worked row's scale is fl32(127/3) = 42.333332..."""
    x = np.array([[0.4, -1.2, 3.0, 0.1]], dtype=np.float16)
    _, c_x, _ = oracle.quantize_rowwise(x, np.zeros(0, np.int32))
    assert Fraction(float(c_x[0])) == rational.fl32(Fraction(127, 3))


@pytest.mark.parametrize("ill", _golden()["tensor_illustrations"], ids=lambda c: c["name"])
def test_tensor_illustrations(ill):
    """[DIGEST] 'Quantization Primitives' (60 among [-3,3] maps to [-6.35, 6.35])
    and [PY] '量化为什么会崩' (100 among +-1: step 0.79, value 1 spans ~1.3 steps)."""
    c = float(oracle.row_scales(np.array([ill["absmax"]], np.float32))[0])
    if "mapped_range_printed" in ill:
        assert round(c * ill["range_max"], 2) == pytest.approx(ill["mapped_range_printed"])
        assert round(c, 2) == pytest.approx(ill["scale_printed"])
    if "step_printed" in ill:
        assert round(1.0 / c, 2) == pytest.approx(ill["step_printed"])
        assert round(ill["range_max"] * c, 1) == pytest.approx(ill["steps_of_value_one_printed"])


# ---------------------------------------------------------------- closed forms

def test_roundtrip_error_bound():
    """[TM] 'Absmax INT8 quantization from first principles': the error per
    element is at most half a step, absmax/254 (non-outlier columns). The
    fp32 product v = fl32(x c) can move a value across a .5 boundary by half
    an fp32 ulp of v (<= 2**-18 for |v| <= 127), so the bound carries a
    relative slack of 2**-16."""
    rng = np.random.default_rng(1)
    X = np.clip(rng.standard_normal((64, 512)) * rng.uniform(0.001, 1.5, (64, 1)), -5.9, 5.9).astype(np.float16)
    X[:, 7] = 40.0
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    Xq, c_x, _ = oracle.quantize_rowwise(X, idx)
    keep = np.ones(512, bool)
    keep[idx] = False
    X64 = X.astype(np.float64)
    m = np.abs(X64[:, keep]).max(axis=1)
    err = np.abs(X64[:, keep] - Xq[:, keep] / c_x[:, None].astype(np.float64))
    assert (err <= (m / 254.0)[:, None] * (1 + 2.0 ** -16)).all()


def test_every_fp16_absmax_maps_to_127():
    """[DIGEST] 'Quantization Primitives', 'What it computes': the
    largest-magnitude value maps to +-127. Checked for every positive finite
    fp16 absmax (the row [m] and the row [-m])."""
    allm = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    X = np.concatenate([allm, -allm])[:, None]
    Xq, c_x, _ = oracle.quantize_rowwise(X, np.zeros(0, np.int32))
    n = allm.size
    assert (Xq[:n, 0] == 127).all()
    assert (Xq[n:, 0] == -127).all()


def test_range_is_symmetric_no_minus_128():
    """[TM]: Q(x) lies in {-127, ..., 127}."""
    rng = np.random.default_rng(2)
    X = (rng.standard_normal((256, 256)) * 3).astype(np.float16)
    _, idx, _ = oracle.outlier_columns(X, INF)
    Xq, _, _ = oracle.quantize_rowwise(X, idx)
    assert Xq.min() >= -127 and Xq.max() <= 127
    W = (rng.standard_normal((256, 128)) * 0.02).astype(np.float16)
    Wq_t, _ = oracle.quantize_colwise_weights(W)
    assert Wq_t.min() >= -127 and (np.abs(Wq_t).max(axis=1) == 127).all()


# ---------------------------------------------------------------- ties and thresholds

@pytest.mark.parametrize("x,expected", [
    (0.00439453125, 1),      # 127*x/m == 0.5 exactly, also in fp32
    (-0.00439453125, -1),
    (0.02197265625, 3),      # == 2.5 exactly
    (-0.02197265625, -3),
])
def test_round_half_away_on_exact_ties(x, expected):
    """Reading: ties round away from zero. These (m, x) fp16 pairs give an
    exact .5 after v = fl32(x * fl32(127/m)); half-to-even would give 0 / 2."""
    m = 1.1162109375
    X = np.array([[m, x]], dtype=np.float16)
    Xq, c_x, _ = oracle.quantize_rowwise(X, np.zeros(0, np.int32))
    v = rational.fl32(Fraction(x) * rational.fl32(Fraction(127) / Fraction(m)))
    assert v.denominator == 2                      # an exact tie
    assert Xq[0, 1] == expected
    assert rational.half_away(v) == expected


def test_alpha_tie_is_outlier():
    """Reading '>=': a column whose largest magnitude is exactly 6.0 is in O
    ([DIGEST] 'The Full LLM.int8() Algorithm', Step 1); the next smaller fp16
    value 5.99609375 is not."""
    X = np.zeros((3, 64), np.float16)
    X[1, 5] = 6.0
    X[2, 9] = -6.0
    X[0, 11] = 5.99609375
    X[2, 40] = -5.99609375
    mask, idx, n = oracle.outlier_columns(X, 6.0)
    assert idx.tolist() == [5, 9]
    assert n == 2
    assert mask.tolist() == [(1 << 5) | (1 << 9), 0]


def test_outlier_set_is_elementwise_with_nan():
    """[DIGEST] 'The Full LLM.int8() Algorithm', Step 1: a column is in O when
    one of its elements reaches alpha. A NaN in the same column must not hide
    that element, and a NaN alone does not reach alpha (brute force over the
    elements in plain Python)."""
    X = np.zeros((4, 64), np.float16)
    X[0, 3] = np.nan
    X[2, 3] = 10.0            # NaN and an outlier: in O
    X[1, 7] = np.nan          # NaN only: not in O
    X[3, 20] = -np.nan
    X[0, 20] = 5.99609375     # NaN and a near miss: not in O
    X[3, 33] = -6.0           # plain outlier: in O
    _, idx, n = oracle.outlier_columns(X, 6.0)
    brute = [j for j in range(64) if any(abs(float(X[i, j])) >= 6.0 for i in range(4))]
    assert brute == [3, 33]
    assert idx.tolist() == brute and n == 2


def test_outlier_column_excluded_from_row_absmax():
    """[DIGEST] Step 4: the row constant is over X^{not O} only. In row 1 the
    outlier column holds 2.0 (< alpha) but it must not set the row absmax."""
    X = np.array([[7.0, 1.0, 0.5, 0.25],
                  [2.0, 1.0, 0.5, -0.25]], np.float16)
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    assert idx.tolist() == [0]
    Xq, c_x, X_O = oracle.quantize_rowwise(X, idx)
    assert c_x.tolist() == [127.0, 127.0]
    assert Xq.tolist() == [[0, 127, 64, 32], [0, 127, 64, -32]]
    assert X_O[:, 0].tolist() == [7.0, 2.0]


def test_zero_row_convention():
    """Convention (parity unpinned: the pages are silent): an all-zero regular
    row gets c_x = 1 and quantises to zeros, contributing nothing."""
    X = np.zeros((2, 64), np.float16)
    X[0, 3] = 9.0
    X[1, 4] = 0.5
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    Xq, c_x, _ = oracle.quantize_rowwise(X, idx)
    assert c_x[0] == 1.0 and not Xq[0].any()
    assert Xq[1, 4] == 127


# ---------------------------------------------------------------- special cases

def test_alpha_zero_is_exact_fp16_matmul():
    """alpha = 0 puts every column in O: Xq == 0, c_x == 1 and C reduces to
    the fp16-rounded float64 product X W (textbook matmul)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((24, 192)).astype(np.float16)
    W = (rng.standard_normal((192, 96)) * 0.02).astype(np.float16)
    out = oracle.forward(X, W, alpha=0.0)
    assert out["n_out"] == 192 and not out["Xq"].any() and (out["c_x"] == 1).all()
    ref = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16)
    assert np.array_equal(out["C"].view(np.uint16), ref.view(np.uint16))


def test_no_outliers_equals_pure_vectorwise():
    """With no element >= alpha the result is pure vector-wise int8
    ([DIGEST] 'Vector-wise Quantization'): alpha=6 and alpha=inf agree
    bit-for-bit, and both agree with the exact rational brute force."""
    rng = np.random.default_rng(4)
    X = np.clip(rng.standard_normal((4, 64)), -5, 5).astype(np.float16)
    W = (rng.standard_normal((64, 8)) * 0.02).astype(np.float16)
    a = oracle.forward(X, W, alpha=6.0)
    b = oracle.forward(X, W, alpha=INF)
    assert a["n_out"] == 0 and b["n_out"] == 0
    for k in ("C", "Xq", "c_x"):
        assert np.array_equal(a[k], b[k])
    _, _, _, _, _, _, C = rational.brute_force(X, W, INF)
    got = [[Fraction(float(v)) for v in row] for row in a["C"]]
    assert got == C


# ---------------------------------------------------------------- brute force

def test_int32_accumulator_bruteforce_tiny():
    """C_i32 on the 16x256x512 tiny workload equals integer dot products
    (int64 numpy, no BLAS) and, on sampled entries, pure-Python sums."""
    inp = make_inputs(get_config("tiny"))
    X, W = inp["X"], inp["W"]
    _, idx, _ = oracle.outlier_columns(X, 6.0)
    Xq, _, _ = oracle.quantize_rowwise(X, idx)
    Wq_t, _ = oracle.quantize_colwise_weights(W)
    C = oracle.int8_matmul_i32(Xq, Wq_t)
    ref = Xq.astype(np.int64) @ Wq_t.astype(np.int64).T
    assert np.array_equal(C.astype(np.int64), ref)
    rng = np.random.default_rng(5)
    for _ in range(50):
        i, j = int(rng.integers(16)), int(rng.integers(512))
        assert int(C[i, j]) == sum(int(a) * int(b) for a, b in zip(Xq[i], Wq_t[j]))


@pytest.mark.parametrize("seed,s,h,o,nout", [
    (10, 4, 32, 8, 1), (11, 8, 64, 16, 2), (12, 5, 128, 12, 3), (13, 8, 128, 16, 0), (14, 3, 96, 7, 5),
])
def test_exact_rational_bruteforce(seed, s, h, o, nout):
    """Exact rational evaluation of every step (fl32/fl16 emulated from the
    IEEE definition) agrees with the oracle: O, c_x, Xq, c_w, Wq, C_i32
    exactly; C within one fp16 ulp (and almost always bit-equal)."""
    inp = random_case(seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    # one row exactly at the threshold when there are outliers
    if nout:
        X[0, int(inp["planted"][0])] = np.float16(6.0)
    O, c_x, Xq, c_w, Wq, Ci, C = rational.brute_force(X, W, 6.0)
    out = oracle.forward(X, W, 6.0, keep=True)
    assert out["idx"].tolist() == O
    assert [Fraction(float(v)) for v in out["c_x"]] == c_x
    assert out["Xq"].tolist() == Xq
    assert [Fraction(float(v)) for v in out["c_w"]] == c_w
    assert out["Wq_t"].T.tolist() == Wq
    Ci_or = oracle.int8_matmul_i32(out["Xq"], out["Wq_t"])
    assert Ci_or.tolist() == Ci
    equal = 0
    for i in range(s):
        for j in range(o):
            g = Fraction(float(out["C"][i, j]))
            assert abs(g - C[i][j]) <= rational.ulp16(C[i][j])
            equal += g == C[i][j]
    assert equal >= s * o - 1


def test_fp16_output_rounding_is_single_rne():
    """The float64 -> fp16 cast used for C is round-to-nearest-even from the
    exact value (checked against the rational definition, incl. ties)."""
    rng = np.random.default_rng(6)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 4, 2000),
                           (np.arange(1, 2000) + 0.5) * 2.0 ** -10])
    for v in vals:
        assert Fraction(float(np.float64(v).astype(np.float16))) == rational.fl16(Fraction(float(v)))


# ---------------------------------------------------------------- invariants

def test_permutation_equivariance():
    """Permuting the columns of X together with the rows of W permutes O and
    leaves c_x, C_i32 and C unchanged (the product is a sum over h)."""
    inp = random_case(20, 12, 256, 64, 3)
    X, W = inp["X"], inp["W"]
    perm = np.random.default_rng(7).permutation(256)
    a = oracle.forward(X, W, 6.0, keep=True)
    b = oracle.forward(X[:, perm], W[perm, :], 6.0, keep=True)
    assert sorted(perm[b["idx"]].tolist()) == a["idx"].tolist()
    assert np.array_equal(a["c_x"], b["c_x"])
    Ca = oracle.int8_matmul_i32(a["Xq"], a["Wq_t"])
    Cb = oracle.int8_matmul_i32(b["Xq"], b["Wq_t"])
    assert np.array_equal(Ca, Cb)
    d = np.abs(a["C"].astype(np.float64) - b["C"].astype(np.float64))
    assert (d <= _ulp16(a["C"])).all()


def test_power_of_two_scale_invariance():
    """Scaling a W column (or an X row) by 2^k leaves its int8 codes
    unchanged and scales its constant by 2^-k exactly."""
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((128, 32)) * 0.02).astype(np.float16)
    W2 = W.copy()
    W2[:, 5] = (W2[:, 5].astype(np.float32) * 8).astype(np.float16)
    W2[:, 9] = (W2[:, 9].astype(np.float32) / 4).astype(np.float16)
    q1, c1 = oracle.quantize_colwise_weights(W)
    q2, c2 = oracle.quantize_colwise_weights(W2)
    assert np.array_equal(q1, q2)
    assert c2[5] == c1[5] / 8 and c2[9] == c1[9] * 4
    X = rng.standard_normal((4, 64)).astype(np.float16)
    X2 = X.copy()
    X2[2] = (X2[2].astype(np.float32) * 2).astype(np.float16)
    a = oracle.quantize_rowwise(X, np.zeros(0, np.int32))
    b = oracle.quantize_rowwise(X2, np.zeros(0, np.int32))
    assert np.array_equal(a[0], b[0]) and b[1][2] == a[1][2] / 2


def _closed_form_bound(X, W, out):
    """|C - X W|_ij <= sum_{k not in O} (|w_kj| m_i + |x_ik| m'_j + m_i m'_j / 254) / 254
    + half an fp16 ulp of C, from the per-element bound m/254 of [TM]."""
    X64 = X.astype(np.float64)
    W64 = W.astype(np.float64)
    s, h = X.shape
    keep = np.ones(h, bool)
    keep[out["idx"]] = False
    m = np.abs(X64[:, keep]).max(axis=1) if keep.any() else np.zeros(s)
    mw = np.abs(W64).max(axis=0)
    Xa, Wa = np.abs(X64[:, keep]), np.abs(W64[keep, :])
    bound = (m[:, None] * Wa.sum(axis=0)[None, :] + Xa.sum(axis=1)[:, None] * mw[None, :]
             + keep.sum() * m[:, None] * mw[None, :] / 254.0) / 254.0
    ref = X64 @ W64
    return ref, bound * (1 + 1e-5) + 0.5 * _ulp16(out["C"]) + 1e-12


@pytest.mark.parametrize("name,rows", [("tiny", None), ("opt67b_ffn1_prefill", 64)])
def test_closed_form_error_bound(name, rows):
    """Elementwise error against the exact product stays inside the bound
    derived from the per-element quantisation error (catches transposed
    operands, wrong scale axes, dropped outlier terms)."""
    w = get_config(name)
    inp = make_inputs(w)
    X, W = inp["X"], inp["W"]
    if rows is not None:
        X = X[:rows]
        W = W[:, :1024]
    out = oracle.forward(X, W, w.alpha)
    assert sorted(out["idx"].tolist()) == sorted(inp["planted"].tolist())
    ref, bound = _closed_form_bound(X, W, out)
    err = np.abs(out["C"].astype(np.float64) - ref)
    assert (err <= bound).all()
    # a plausible mistake breaks it: drop the outlier term
    bad = oracle.dequantize_and_add(
        oracle.int8_matmul_i32(out["Xq"], oracle.quantize_colwise_weights(W)[0]),
        out["c_x"], oracle.quantize_colwise_weights(W)[1], None)
    assert (np.abs(bad.astype(np.float64) - ref) > bound).any()


def test_generator_plants_exact_outlier_sets():
    """The generator's planted columns are exactly the detected O (alpha = 6)."""
    for name in ("tiny", "opt67b_ffn1_prefill"):
        inp = make_inputs(get_config(name), with_W=False)
        _, idx, _ = oracle.outlier_columns(inp["X"], 6.0)
        assert idx.tolist() == sorted(inp["planted"].tolist())


@pytest.mark.parametrize("seed,s,h,o", [(11, 3, 64, 8), (12, 5, 128, 4), (13, 2, 192, 6)])
def test_fp16_baseline_is_exact_product_rounded_once(seed, s, h, o):
    """The FP16 baseline of Table 5 ([DIGEST] 'Runtime Performance (Appendix
    D)'): fp16_matmul equals the exact rational product X W rounded once to
    fp16 (round to nearest even, written from the IEEE definition)."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((s, h)).astype(np.float16)
    W = (rng.standard_normal((h, o)) * 0.05).astype(np.float16)
    got = oracle.fp16_matmul(X, W)
    Xf, Wf = rational.to_fractions(X), rational.to_fractions(W)
    for i in range(s):
        for j in range(o):
            exact = sum(Xf[i][k] * Wf[k][j] for k in range(h))
            assert Fraction(float(got[i, j])) == rational.fl16(exact), (i, j)


def test_fp16_baseline_equals_full_decomposition():
    """With alpha = 0 every column is an outlier and the decomposition is the
    plain fp16 product: forward(alpha=0) and fp16_matmul agree bit for bit
    (two independent routes through the oracle)."""
    rng = np.random.default_rng(14)
    X = rng.standard_normal((9, 320)).astype(np.float16)
    W = (rng.standard_normal((320, 40)) * 0.02).astype(np.float16)
    a = oracle.fp16_matmul(X, W, col_chunk=16)
    b = oracle.forward(X, W, alpha=0.0)["C"]
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def _lossless_weights(rng, h, o):
    """W whose column-wise int8 quantisation is exact: per column an integer
    code vector with max |q| = 127 times a power-of-two scale 2^-e, so
    c_w = 2^e exactly and W_i8 / c_w == W."""
    q = rng.integers(-127, 128, size=(h, o))
    q[rng.integers(0, h, size=o), np.arange(o)] = 127
    e = rng.integers(5, 9, size=o)
    return (q * np.exp2(-e)[None, :]).astype(np.float16)


def test_rebuilt_outlier_rows_equal_fp16_rows_when_lossless():
    """Without a resident fp16 W the outlier rows are W_i8 / c_w; for weights
    whose quantisation is lossless the two storage variants give the same
    C bit for bit (a wrong row, column or scale in the rebuild would not)."""
    rng = np.random.default_rng(21)
    inp = random_case(21, 12, 256, 96, 4, row_frac=0.5)
    W = _lossless_weights(rng, 256, 96)
    Wq_t, c_w = oracle.quantize_colwise_weights(W)
    assert np.array_equal((Wq_t.T.astype(np.float64) / c_w[None, :]).astype(np.float16), W)
    a = oracle.forward(inp["X"], W, 6.0)
    b = oracle.forward(inp["X"], W, 6.0, fp16_weights=False)
    assert a["n_out"] == 4
    assert np.array_equal(a["C"].view(np.uint16), b["C"].view(np.uint16))


def test_rebuilt_outlier_rows_are_rounded_products_with_the_inverse_scale():
    """Each rebuilt weight is fl16(fl32(code * fl32(1 / c_w))), every rounding
    emulated from its IEEE definition with rational arithmetic, for ordinary
    weights; and it lies within one fp16 ulp (plus the two fp32 roundings)
    of the exact quotient code / c_w, i.e. of the dequantised value."""
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((64, 24)) * 0.02).astype(np.float16)
    Wq_t, c_w = oracle.quantize_colwise_weights(W)
    idx = np.array([3, 17, 40, 63])
    rows = oracle.dequantized_outlier_rows(Wq_t, c_w, idx)
    for a, k in enumerate(idx):
        for j in range(24):
            q = Fraction(int(Wq_t[j, k]))
            inv = rational.fl32(1 / Fraction(float(c_w[j])))
            got = Fraction(float(rows[a, j]))
            assert got == rational.fl16(rational.fl32(q * inv))
            assert abs(got - q / Fraction(float(c_w[j]))) <= rational.ulp16(got) * (1 + Fraction(1, 1 << 20))


# ---------------------------------------------------------------- layer bias

def test_bias_alone_with_zero_weights():
    """W = 0 (every code 0, c_w = 1 by the zero-column convention): C is the
    bias broadcast over the rows, bit for bit, whatever X holds (outlier
    columns included). A bias dropped, doubled or indexed by row fails."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((6, 128)).astype(np.float16)
    X[:, 5] = 9.0
    W = np.zeros((128, 64), np.float16)
    b = (rng.standard_normal(64) * 3).astype(np.float16)
    out = oracle.forward(X, W, 6.0, bias=b)
    assert out["n_out"] == 1
    assert np.array_equal(out["C"].view(np.uint16), np.broadcast_to(b, (6, 64)).view(np.uint16))


def test_bias_alpha_zero_is_textbook_linear_layer():
    """alpha = 0 (no int8 part): C is the fp16-rounded float64 X W + b, the
    textbook linear layer."""
    rng = np.random.default_rng(32)
    X = rng.standard_normal((20, 128)).astype(np.float16)
    W = (rng.standard_normal((128, 80)) * 0.02).astype(np.float16)
    b = rng.standard_normal(80).astype(np.float16)
    out = oracle.forward(X, W, alpha=0.0, bias=b)
    ref = (X.astype(np.float64) @ W.astype(np.float64) + b.astype(np.float64)[None, :]).astype(np.float16)
    assert np.array_equal(out["C"].view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("seed,s,h,o,nout", [(40, 4, 64, 12, 2), (41, 6, 128, 8, 0)])
def test_bias_exact_rational_bruteforce(seed, s, h, o, nout):
    """With a bias, C agrees with the exact rational evaluation of every step
    plus b_j, rounded once (within one fp16 ulp, almost always bit-equal)."""
    inp = random_case(seed, s, h, o, nout, row_frac=0.5)
    b = (np.random.default_rng(seed).standard_normal(o) * 0.5).astype(np.float16)
    *_, C = rational.brute_force(inp["X"], inp["W"], 6.0, bias=b)
    out = oracle.forward(inp["X"], inp["W"], 6.0, bias=b)
    equal = 0
    for i in range(s):
        for j in range(o):
            g = Fraction(float(out["C"][i, j]))
            assert abs(g - C[i][j]) <= rational.ulp16(C[i][j])
            equal += g == C[i][j]
    assert equal >= s * o - 1
