"""GPU parity of every C-ABI entry point against the CPU oracle on seeded
inputs small enough for the oracle to finish in seconds, spanning several
tiles and ragged tails of both main loops (s <= 16 weight streaming, s > 16
LDS-tiled), plus the method's degenerate cases.

Bars: bit-exact for the outlier set, int8 codes, fp32 scales, gathered
outlier columns and int32 accumulators; max |C - C_ref| <= 2e-3 ||C_ref||_inf
for the fp16 output.
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, check_rows, round_up, say
from workloads import get_config, make_inputs, random_case

pytestmark = pytest.mark.gpu

# (seed, s, h, o, n_outliers, row_frac): ragged s, o tails vs the 256 tiles,
# h % 128 == 64 K tails, decode (s <= 16) and prefill main loops.
SHAPES = [
    (0, 1, 64, 64, 0, 0.0),
    (1, 5, 192, 128, 2, 1.0),
    (2, 16, 256, 512, 2, 0.3),
    (3, 17, 192, 320, 3, 0.5),
    (4, 64, 512, 1024, 7, 0.75),
    (5, 300, 640, 576, 5, 0.06),
    (6, 513, 384, 768, 40, 0.28),
    (7, 8, 1024, 1024, 64, 1.0),
    (8, 257, 1152, 832, 1, 1.0),
    (9, 40, 64, 320, 1, 0.5),        # one panel: the only K stage is half empty
    (10, 300, 1088, 448, 3, 0.3),    # 8.5 K stages; o past one 256-column tile
    (11, 16, 1088, 448, 3, 0.3),     # the same shape on the streaming path
]


def _run_all(X, W, alpha):
    Xd, Wd = T(X), T(W)
    say(f"  launch: detect/quantize/gemm s={X.shape[0]} h={X.shape[1]} o={W.shape[1]} alpha={alpha}")
    mask, idx, n_out = i8.detect_outlier_cols(Xd, alpha)
    Xq, c_x, X_O = i8.quantize_rowwise(Xd, mask, idx, n_out)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    C = i8.int8_mixed_matmul(Xq, c_x, X_O, idx, n_out, Wq, c_w, Wd)
    Ci = i8.int8_gemm_i32(Xq, Wq)
    CO = i8.outlier_matmul(X_O, idx, n_out, Wd)
    torch.cuda.synchronize()
    return dict(mask=mask, idx=idx, n_out=n_out, Xq=Xq, c_x=c_x, X_O=X_O, Wq=Wq, c_w=c_w, C=C, Ci=Ci, CO=CO)


def _check_all(X, W, alpha, g):
    idx_r = check_detect(X, alpha, g["mask"], g["idx"], g["n_out"])
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, g["Xq"], g["c_x"], g["X_O"])
    Wq_r, cw_r = oracle.quantize_colwise_weights(W)
    assert np.array_equal(H(i8.panels_to_rows(g["Wq"])), Wq_r), "Wq differs"
    assert np.array_equal(H(g["c_w"]).view(np.uint32), cw_r.view(np.uint32)), "c_w differs"
    Ci_r = oracle.int8_matmul_i32(Xq_r, Wq_r)
    assert np.array_equal(H(g["Ci"]), Ci_r), "C_i32 differs"
    CO_r = oracle.outlier_matmul(XO_r, W, idx_r)
    CO = H(g["CO"]).astype(np.float64)
    scale = np.abs(XO_r.astype(np.float64)) @ np.abs(W[idx_r].astype(np.float64)) if idx_r.size else 0.0
    assert (np.abs(CO - CO_r) <= 1e-5 * scale + 1e-30).all(), "outlier product differs"
    C_r = oracle.int8_mixed_matmul(Xq_r, cx_r, XO_r, idx_r, Wq_r, cw_r, W)
    return check_C(g["C"], C_r)


@pytest.mark.parametrize("seed,s,h,o,nout,frac", SHAPES, ids=[f"s{c[1]}h{c[2]}o{c[3]}n{c[4]}" for c in SHAPES])
def test_all_entry_points_match_oracle(seed, s, h, o, nout, frac):
    inp = random_case(seed, s, h, o, nout, row_frac=frac)
    X, W = inp["X"], inp["W"]
    if nout:
        X[0, int(inp["planted"][0])] = np.float16(6.0)   # an element exactly at alpha
    g = _run_all(X, W, 6.0)
    rel = _check_all(X, W, 6.0, g)
    say(f"  max rel err {rel:.2e}")


def test_tiny_config():
    w = get_config("tiny")
    inp = make_inputs(w)
    g = _run_all(inp["X"], inp["W"], w.alpha)
    assert int(H(g["n_out"])[0]) == 2
    _check_all(inp["X"], inp["W"], w.alpha, g)


@pytest.mark.parametrize("s", [12, 40])
def test_alpha_zero_every_column_is_outlier(s):
    """alpha = 0: O = all columns, Xq == 0, C == fp16(X W) from the fp16 MFMA path."""
    inp = random_case(30 + s, s, 128, 192, 0)
    X, W = inp["X"], inp["W"]
    g = _run_all(X, W, 0.0)
    assert int(H(g["n_out"])[0]) == 128
    assert not H(g["Xq"]).any()
    _check_all(X, W, 0.0, g)
    ref = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16)
    check_C(g["C"], ref)


@pytest.mark.parametrize("s", [4, 33])
def test_alpha_inf_is_pure_vectorwise(s):
    inp = random_case(40 + s, s, 256, 256, 3)
    g = _run_all(inp["X"], inp["W"], float("inf"))
    assert int(H(g["n_out"])[0]) == 0
    _check_all(inp["X"], inp["W"], float("inf"), g)


@pytest.mark.parametrize("s", [3, 20])
def test_zero_rows_and_zero_input(s):
    inp = random_case(50 + s, s, 128, 128, 1, row_frac=0.5)
    X = inp["X"]
    X[1, :] = 0                      # an all-zero row
    X[2, :] = 0
    X[2, int(inp["planted"][0])] = 9.0   # a row whose only non-zero is an outlier
    g = _run_all(X, inp["W"], 6.0)
    _check_all(X, inp["W"], 6.0, g)
    Z = np.zeros_like(X)
    g = _run_all(Z, inp["W"], 6.0)
    assert not H(g["C"]).view(np.uint16).any()
    assert (H(g["c_x"]) == 1.0).all()


@pytest.mark.parametrize("s", [2, 17])
def test_max_h_int32_accumulator_bound(s):
    """h = 133120 (largest accepted): all codes 127 give C_i32 = h * 127^2,
    just below 2^31, exactly (C = h / 4 stays finite in fp16)."""
    h, o = 133120, 64
    X = np.ones((s, h), np.float16)
    W = np.full((h, o), 0.25, np.float16)
    Xd, Wd = T(X), T(W)
    say(f"  launch: max-h s={s}")
    mask, idx, n_out = i8.detect_outlier_cols(Xd, 6.0)
    Xq, c_x, X_O = i8.quantize_rowwise(Xd, mask, idx, n_out)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    Ci = i8.int8_gemm_i32(Xq, Wq)
    C = i8.int8_mixed_matmul(Xq, c_x, X_O, idx, n_out, Wq, c_w, Wd)
    torch.cuda.synchronize()
    assert int(H(n_out)[0]) == 0
    assert (H(Ci) == h * 127 * 127).all()
    assert h * 127 * 127 < 2 ** 31
    check_C(C, (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16))


def test_forward_matches_separate_calls_and_is_deterministic():
    inp = random_case(60, 70, 768, 640, 6, row_frac=0.75)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(70, 768, DEV)
    C1 = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
    v = {k: t.clone() for k, t in i8.forward_workspace_views(ws, 70, 768).items()}
    C2 = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    g = _run_all(X, W, 6.0)
    assert torch.equal(g["C"], C1)
    n = int(H(v["n_out"])[0])
    assert torch.equal(v["idx"][:n], g["idx"][:n]) and torch.equal(v["mask"], g["mask"])
    assert torch.equal(v["Xq"], g["Xq"]) and torch.equal(v["c_x"], g["c_x"])


# Forward paths: s <= 8 runs the slab kernels (one row group of 16), larger s
# the accumulator path (detection, then one to four wavefronts per row, the
# row held in registers for h <= 32768 and re-read above); the products: the
# K-split weight stream up to 16 rows, the column-split one up to 128 rows,
# the tiled one above.
# (70, 768) once overran a former single-block path's 16-row tables.
FWD = [(70, 768, 640, 6, 6.0), (16, 8192, 256, 7, 6.0), (17, 8192, 256, 7, 6.0), (33, 1024, 256, 7, 6.0),
       (64, 2048, 256, 7, 6.0), (65, 2048, 256, 7, 6.0), (300, 640, 576, 5, 6.0),
       (8, 16384, 128, 9, 6.0), (9, 12288, 128, 9, 6.0), (66, 16384, 128, 9, 6.0), (70, 20480, 128, 9, 6.0),
       (3, 133120, 64, 9, 6.0),
       (40, 128, 192, 0, 0.0), (1100, 128, 192, 0, 0.0), (513, 384, 768, 40, 6.0), (2, 64, 64, 0, 6.0),
       (1, 16384, 128, 5, 6.0), (5, 8256, 192, 3, 6.0), (12, 8192, 256, 0, 6.0), (10, 4096, 128, 0, 0.0),
       (16, 64, 64, 2, 6.0), (8, 12288, 256, 7, float("inf")), (7, 1024, 128, 64, 6.0)]


@pytest.mark.parametrize("s,h,o,nout,alpha", FWD, ids=[f"s{c[0]}h{c[1]}n{c[3]}a{c[4]}" for c in FWD])
def test_forward_paths_match_separate_calls(s, h, o, nout, alpha):
    inp = random_case(70 + s, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    say(f"  launch: forward s={s} h={h} o={o} alpha={alpha}")
    C1 = i8.forward(Xd, Wq, c_w, Wd, alpha, workspace=ws)
    torch.cuda.synchronize()
    v = {k: t.clone() for k, t in i8.forward_workspace_views(ws, s, h).items()}
    assert not v["acc"].any(), "accumulator not returned to zero"
    g = _run_all(X, W, alpha)
    n = int(H(g["n_out"])[0])
    assert int(H(v["n_out"])[0]) == n
    assert torch.equal(v["mask"], g["mask"]) and torch.equal(v["idx"][:n], g["idx"][:n])
    assert torch.equal(v["Xq"], g["Xq"]) and torch.equal(v["c_x"], g["c_x"])
    npad = round_up(n, 32)
    assert torch.equal(v["X_O"][:, :npad], g["X_O"][:, :npad])
    assert torch.equal(C1, g["C"])
    _check_all(X, W, alpha, dict(g, mask=v["mask"], idx=v["idx"], n_out=v["n_out"], Xq=v["Xq"], c_x=v["c_x"],
                                 X_O=v["X_O"], C=C1))
    C2 = i8.forward(Xd, Wq, c_w, Wd, alpha, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_forward_workspace_reuse_across_shapes():
    """One workspace, shapes alternating between the two prologue paths
    (few rows: slabs of 128 columns, one and four groups of 16 rows; many
    rows: detection then rows)."""
    big = i8.forward_workspace(1100, 640, DEV)
    for (s, h, o, nout) in [(1100, 640, 256, 5), (8, 640, 256, 3), (40, 640, 256, 4), (600, 640, 320, 9),
                            (8, 640, 256, 3), (40, 640, 256, 4)]:
        inp = random_case(90 + s + nout, s, h, o, nout, row_frac=0.5)
        X, W = inp["X"], inp["W"]
        Xd, Wd = T(X), T(W)
        Wq, c_w = i8.quantize_colwise_weights(Wd)
        say(f"  launch: forward reuse s={s} h={h}")
        C = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=big)
        torch.cuda.synchronize()
        ref = _run_all(X, W, 6.0)
        assert torch.equal(C, ref["C"])
        assert not i8.forward_workspace_views(big, s, h)["acc"].any()


def test_bad_arguments_raise():
    X = torch.zeros((4, 96), dtype=torch.float16, device=DEV)
    with pytest.raises(i8.I8MMError):
        i8.detect_outlier_cols(X)
    with pytest.raises(ValueError):
        i8.detect_outlier_cols(torch.zeros((4, 64), dtype=torch.float32, device=DEV))


# Dense fp16 baseline (Table 5's FP16 reference): packing is a pure layout
# change (exact); the product is checked against the oracle's fp16(X W).
FP16 = [(1, 64, 64), (17, 192, 320), (40, 64, 320), (300, 1088, 448), (513, 384, 768), (16, 1024, 512)]


@pytest.mark.parametrize("s,h,o", FP16, ids=[f"s{c[0]}h{c[1]}o{c[2]}" for c in FP16])
def test_fp16_gemm_matches_oracle(s, h, o):
    rng = np.random.default_rng(s + h + o)
    X = rng.standard_normal((s, h)).astype(np.float16)
    W = (rng.standard_normal((h, o)) * 0.02).astype(np.float16)
    Xd, Wd = T(X), T(W)
    say(f"  launch: fp16 pack + gemm s={s} h={h} o={o}")
    Wp = i8.pack_fp16_weights(Wd)
    C = i8.fp16_gemm(Xd, Wp)
    torch.cuda.synchronize()
    assert np.array_equal(H(Wp).transpose(1, 0, 2).reshape(o, h), W.T)
    check_C(C, oracle.fp16_matmul(X, W))
    C2 = i8.fp16_gemm(Xd, Wp)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)


def test_fp16_gemm_full_size_sampled():
    """The 2048 x 4096 x 16384 layer of the prefill benchmark, sampled rows x
    columns against the oracle."""
    s, h, o = 2048, 4096, 16384
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    Xd = torch.randn((s, h), generator=g, device=DEV).half()
    Wd = (0.02 * torch.randn((h, o), generator=g, device=DEV)).half()
    say("  launch: fp16 pack + gemm 2048x4096x16384")
    Wp = i8.pack_fp16_weights(Wd)
    C = i8.fp16_gemm(Xd, Wp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, s - 1], rng.choice(s, 30, replace=False)]))
    cols = np.unique(np.concatenate([[0, o - 1], rng.choice(o, 200, replace=False)]))
    X, W = H(Xd), H(Wd)
    ref = oracle.fp16_matmul(X[rows], W[:, cols])
    check_C(C.index_select(0, torch.from_numpy(rows).to(DEV)).index_select(1, torch.from_numpy(cols).to(DEV)), ref)


# Without a resident fp16 W (W = None): outlier rows rebuilt from W_i8 / c_w.
W8 = [(70, 768, 640, 6), (300, 1088, 448, 40), (600, 512, 768, 100), (8, 1024, 512, 3), (9, 12288, 128, 9)]


@pytest.mark.parametrize("s,h,o,nout", W8, ids=[f"s{c[0]}h{c[1]}n{c[3]}" for c in W8])
def test_forward_without_fp16_weights(s, h, o, nout):
    inp = random_case(110 + s, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    say(f"  launch: forward without fp16 W s={s} h={h} o={o} |O|={nout}")
    C = i8.forward(Xd, Wq, c_w, None, 6.0, workspace=ws)
    torch.cuda.synchronize()
    v = i8.forward_workspace_views(ws, s, h)
    C2 = i8.int8_mixed_matmul(v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w, None)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    assert not v["acc"].any()
    check_C(C, oracle.forward(X, W, 6.0, fp16_weights=False)["C"])


@pytest.mark.parametrize("s", [8, 300])
def test_without_fp16_weights_is_exact_for_lossless_weights(s):
    """When W_i8 / c_w reproduces W exactly, dropping the fp16 W changes nothing:
    both storage variants give bit-identical C (decode and prefill kernels)."""
    h, o = 512, 384
    rng = np.random.default_rng(s)
    q = rng.integers(-127, 128, size=(h, o))
    q[rng.integers(0, h, size=o), np.arange(o)] = 127
    W = (q * np.exp2(-rng.integers(5, 9, size=o))[None, :]).astype(np.float16)
    X = random_case(120 + s, s, h, o, 5, row_frac=0.5)["X"]
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    say(f"  launch: lossless weights s={s}")
    C1 = i8.forward(Xd, Wq, c_w, Wd, 6.0)
    C2 = i8.forward(Xd, Wq, c_w, None, 6.0)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


# The layer bias (fp16 [o]) added in the epilogue before the one rounding:
# decode and prefill kernels, fp16 W resident or rebuilt, the prefill
# epilogue's single-pass (|O| <= 96) and multi-round outlier paths.
BIAS = [(8, 1024, 512, 3, True), (8, 1024, 512, 3, False), (70, 768, 640, 6, True),
        (300, 1088, 448, 100, True), (300, 1088, 448, 100, False), (17, 192, 320, 0, True)]


@pytest.mark.parametrize("s,h,o,nout,fp16_w", BIAS, ids=[f"s{c[0]}h{c[1]}n{c[3]}{'w' if c[4] else 'q'}" for c in BIAS])
def test_forward_with_bias(s, h, o, nout, fp16_w):
    inp = random_case(130 + s + nout, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    b = (np.random.default_rng(s + o).standard_normal(o) * 0.5).astype(np.float16)
    Xd, Wd, bd = T(X), T(W), T(b)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    say(f"  launch: forward with bias s={s} h={h} o={o} |O|={nout} fp16 W={fp16_w}")
    C = i8.forward(Xd, Wq, c_w, Wd if fp16_w else None, 6.0, workspace=ws, bias=bd)
    torch.cuda.synchronize()
    v = i8.forward_workspace_views(ws, s, h)
    C2 = i8.int8_mixed_matmul(v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w,
                              Wd if fp16_w else None, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    check_C(C, oracle.forward(X, W, 6.0, fp16_weights=fp16_w, bias=b)["C"])


@pytest.mark.parametrize("s", [5, 260])
def test_bias_alone_with_zero_weights(s):
    """W = 0: every row of C is the bias, bit for bit (a bias read at the wrong
    column, or from the row index, cannot pass)."""
    h, o = 256, 576
    X = random_case(140 + s, s, h, o, 2, row_frac=0.5)["X"]
    b = (np.random.default_rng(s).standard_normal(o) * 3).astype(np.float16)
    Wd = torch.zeros((h, o), dtype=torch.float16, device=DEV)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    say(f"  launch: zero weights with bias s={s}")
    C = i8.forward(T(X), Wq, c_w, Wd, 6.0, bias=T(b))
    torch.cuda.synchronize()
    assert np.array_equal(H(C).view(np.uint16), np.broadcast_to(b, (s, o)).view(np.uint16))


@pytest.mark.parametrize("s,h", [(12, 256), (40, 64), (70, 256)])
def test_rebuilt_outlier_rows_bit_exact(s, h):
    """Without a resident fp16 W, at alpha = 0 (every column in O, Xq = 0)
    and with one-hot rows of X, row i of C is the rebuilt weight row of its
    one column, fl16(fl32(q * fl32(1 / c_w))), which must match the
    oracle's bit for bit (decode kernel; prefill single-pass and
    multi-round outlier epilogues)."""
    o = 320
    rng = np.random.default_rng(s + h)
    W = (rng.standard_normal((h, o)) * 0.02).astype(np.float16)
    cols = rng.choice(h, size=s, replace=s > h)
    X = np.zeros((s, h), np.float16)
    X[np.arange(s), cols] = 1.0
    Wd = T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    say(f"  launch: one-hot rows, rebuilt outlier rows s={s} h={h}")
    C = i8.forward(T(X), Wq, c_w, None, 0.0)
    torch.cuda.synchronize()
    Wq_t, cw_r = oracle.quantize_colwise_weights(W)
    ref = oracle.dequantized_outlier_rows(Wq_t, cw_r, cols)
    assert np.array_equal(H(C).view(np.uint16), ref.view(np.uint16))
