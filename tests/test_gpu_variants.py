"""GPU parity of the quantiser variants (tensor-wise, row-wise, zeropoint
vector-wise; [DIGEST] "Quantization Primitives" and "Vector-wise
Quantization", Table 1) against the CPU oracle, through the C ABI.

Bars: bit-exact for the codes, constants, zero points, code sums and the
gathered outlier columns; max |C - C_ref| <= 2e-3 ||C_ref||_inf for C.
Shapes cover the weight-streaming (s <= 16) and LDS-tiled products, ragged
tiles, no decomposition (alpha = inf), and more outlier columns than the
prefill epilogue stages at once.
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, round_up, say
from workloads import random_case

pytestmark = pytest.mark.gpu

# (seed, s, h, o, n_outliers, alpha)
SHAPES = [(0, 8, 1024, 512, 3, 6.0), (1, 300, 1088, 448, 5, 6.0), (2, 17, 192, 320, 2, 6.0),
          (3, 40, 512, 256, 0, float("inf")), (4, 260, 640, 576, 100, 6.0), (5, 5, 12288, 128, 7, 6.0),
          (6, 64, 704, 192, 4, 6.0)]
IDS = [f"s{c[1]}h{c[2]}n{c[4]}a{c[5]}" for c in SHAPES]


def _gpu_detect(X, alpha):
    mask, idx, n_out = i8.detect_outlier_cols(T(X), alpha)
    torch.cuda.synchronize()
    return mask, idx, n_out, check_detect(X, alpha, mask, idx, n_out)


def _check_XO(XO_d, XO_r):
    n = XO_r.shape[1]
    XO = H(XO_d)
    assert np.array_equal(XO[:, :n].view(np.uint16), XO_r.view(np.uint16)), "X_O differs"
    assert not XO[:, n:round_up(n, 32)].view(np.uint16).any(), "X_O padding not zero"


@pytest.mark.parametrize("seed,s,h,o,nout,alpha", SHAPES, ids=IDS)
def test_tensorwise_and_rowwise(seed, s, h, o, nout, alpha):
    inp = random_case(200 + seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    say(f"  launch: tensor/row-wise s={s} h={h} o={o} |O|={nout} alpha={alpha}")
    mask, idx, n_out, idx_r = _gpu_detect(X, alpha)
    Xd, Wd = T(X), T(W)
    Xq, c_x, X_O = i8.quantize_tensorwise(Xd, mask, idx, n_out)
    Wq, c_w = i8.quantize_weights_tensorwise(Wd)
    torch.cuda.synchronize()
    Xq_r, cx_r, XO_r = oracle.quantize_tensorwise(X, idx_r)
    assert np.array_equal(H(Xq), Xq_r), "tensor-wise Xq differs"
    assert np.array_equal(H(c_x).view(np.uint32), cx_r.view(np.uint32)), "tensor-wise c_x differs"
    _check_XO(X_O, XO_r)
    Wq_r, cw_r = oracle.quantize_weights_tensorwise(W)
    assert np.array_equal(H(i8.panels_to_rows(Wq)), Wq_r), "tensor-wise Wq differs"
    assert np.array_equal(H(c_w).view(np.uint32), cw_r.view(np.uint32)), "tensor-wise c_w differs"
    for scheme in ("tensor", "row"):
        C = i8.variant_forward(Xd, (Wq, c_w), Wd, scheme, alpha)
        torch.cuda.synchronize()
        check_C(C, oracle.variant_forward(X, W, scheme, alpha))


@pytest.mark.parametrize("seed,s,h,o,nout,alpha", SHAPES, ids=IDS)
def test_zeropoint(seed, s, h, o, nout, alpha):
    inp = random_case(220 + seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"].copy(), inp["W"].copy()
    X[: s // 2] = np.abs(X[: s // 2])                 # one-signed rows: zero points far from 0
    X[s // 2:] += np.float16(1.5)                      # shifted rows
    W[:, : o // 4] = np.abs(W[:, : o // 4])            # one-signed columns
    say(f"  launch: zeropoint s={s} h={h} o={o} |O|={nout} alpha={alpha}")
    mask, idx, n_out, idx_r = _gpu_detect(X, alpha)
    Xd, Wd = T(X), T(W)
    Xq, nd_x, zp_x, rs_x, X_O = i8.quantize_rowwise_zeropoint(Xd, mask, idx, n_out)
    Wq, nd_w, zp_w, cs_w = i8.quantize_colwise_weights_zeropoint(Wd)
    torch.cuda.synchronize()
    Xq_r, ndx_r, zpx_r, XO_r = oracle.quantize_rowwise_zeropoint(X, idx_r)
    assert np.array_equal(H(Xq), Xq_r), "zeropoint Xq differs"
    assert np.array_equal(H(nd_x).view(np.uint32), ndx_r.view(np.uint32)), "nd_x differs"
    assert np.array_equal(H(zp_x), zpx_r), "zp_x differs"
    assert np.array_equal(H(rs_x), Xq_r.astype(np.int64).sum(axis=1)), "rowsum_x differs"
    _check_XO(X_O, XO_r)
    Wq_r, ndw_r, zpw_r = oracle.quantize_colwise_weights_zeropoint(W)
    assert np.array_equal(H(i8.panels_to_rows(Wq)), Wq_r), "zeropoint Wq differs"
    assert np.array_equal(H(nd_w).view(np.uint32), ndw_r.view(np.uint32)), "nd_w differs"
    assert np.array_equal(H(zp_w), zpw_r), "zp_w differs"
    assert np.array_equal(H(cs_w), Wq_r.astype(np.int64).sum(axis=1)), "colsum_w differs"
    C = i8.zeropoint_matmul(Xq, nd_x, zp_x, rs_x, X_O, idx, n_out, Wq, nd_w, zp_w, cs_w, Wd)
    torch.cuda.synchronize()
    check_C(C, oracle.zeropoint_matmul(Xq_r, ndx_r, zpx_r, XO_r, idx_r, Wq_r, ndw_r, zpw_r, W))
    C2 = i8.variant_forward(Xd, (Wq, nd_w, zp_w, cs_w), Wd, "zeropoint", alpha)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)


@pytest.mark.parametrize("s", [8, 300])
def test_zeropoint_on_symmetric_data_equals_absmax(s):
    """Rows and columns whose min is -max: the zeropoint path must give the
    vector-wise absmax path's C bit for bit (zp = 0, nd = the absmax
    constant), in both product kernels."""
    h, o = 512, 384
    inp = random_case(240 + s, s, h, o, 4, row_frac=0.5)
    _, idx_r, _ = oracle.outlier_columns(inp["X"], 6.0)
    X = inp["X"].copy()
    reg = np.setdiff1d(np.arange(h), idx_r)
    m = np.abs(X[:, reg].astype(np.float32)).max(axis=1).astype(np.float16)
    X[:, reg[0]], X[:, reg[1]] = m, -m
    W = inp["W"].copy()
    mw = np.abs(W.astype(np.float32)).max(axis=0).astype(np.float16)
    W[0], W[1] = mw, -mw
    Xd, Wd = T(X), T(W)
    say(f"  launch: zeropoint vs absmax on symmetric data s={s}")
    Cz = i8.variant_forward(Xd, i8.quantize_weights(Wd, "zeropoint"), Wd, "zeropoint")
    Cv = i8.variant_forward(Xd, i8.quantize_weights(Wd, "vector"), Wd, "vector")
    torch.cuda.synchronize()
    assert torch.equal(Cz, Cv)


@pytest.mark.parametrize("s", [8, 300])
def test_variants_with_bias(s):
    h, o = 640, 320
    inp = random_case(250 + s, s, h, o, 3, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    b = (np.random.default_rng(s).standard_normal(o) * 0.5).astype(np.float16)
    Xd, Wd, bd = T(X), T(W), T(b)
    for scheme in i8.SCHEMES:
        say(f"  launch: {scheme} with bias s={s}")
        C = i8.variant_forward(Xd, i8.quantize_weights(Wd, scheme), Wd, scheme, bias=bd)
        torch.cuda.synchronize()
        check_C(C, oracle.variant_forward(X, W, scheme, bias=b))


# (s, h): every launch shape of the zeropoint row quantiser, named by the
# wavefronts per row and chunks per lane it picks (more rows, fewer
# wavefronts per row; rows longer than 16 chunks per lane take the two-pass
# kernel that reads each row twice).
ZP_ROW_SHAPES = [(2048, 256, "W2 CPL2"), (2048, 4096, "W2 CPL4"), (2048, 8192, "W2 CPL8"),
                 (4096, 256, "W1 CPL2"), (4096, 2048, "W1 CPL4"), (64, 8192, "W4 CPL4"),
                 (16, 16384, "W4 CPL8"), (4, 32768, "W4 CPL16"), (3, 40960, "two-pass")]


@pytest.mark.parametrize("s,h,label", ZP_ROW_SHAPES, ids=[c[2] for c in ZP_ROW_SHAPES])
def test_zeropoint_rows_every_launch_shape(s, h, label):
    inp = random_case(260 + s % 97 + h % 89, s, h, 64, 5, row_frac=0.5)
    X = inp["X"].copy()
    X[: s // 2] = np.abs(X[: s // 2])                  # one-signed rows
    X[s // 2:] += np.float16(1.5)                       # shifted rows
    say(f"  launch: zeropoint rows {label} s={s} h={h}")
    mask, idx, n_out, idx_r = _gpu_detect(X, 6.0)
    Xq, nd_x, zp_x, rs_x, X_O = i8.quantize_rowwise_zeropoint(T(X), mask, idx, n_out)
    torch.cuda.synchronize()
    Xq_r, ndx_r, zpx_r, XO_r = oracle.quantize_rowwise_zeropoint(X, idx_r)
    assert np.array_equal(H(Xq), Xq_r), "zeropoint Xq differs"
    assert np.array_equal(H(nd_x).view(np.uint32), ndx_r.view(np.uint32)), "nd_x differs"
    assert np.array_equal(H(zp_x), zpx_r), "zp_x differs"
    assert np.array_equal(H(rs_x), Xq_r.astype(np.int64).sum(axis=1)), "rowsum_x differs"
    _check_XO(X_O, XO_r)


# (s, h): launch shapes of the tensor-wise row passes (row maxima, then codes
# with the one constant): few rows split over 4 wavefronts with the row in
# registers at 2 to 16 chunks per lane, otherwise one wavefront per row.
TW_ROW_SHAPES = [(8, 1024, "W4 CPL2"), (64, 8192, "W4 CPL4"), (16, 16384, "W4 CPL8"), (4, 32768, "W4 CPL16"),
                 (3, 40960, "one wavefront per row"), (2048, 256, "many rows")]


@pytest.mark.parametrize("s,h,label", TW_ROW_SHAPES, ids=[c[2] for c in TW_ROW_SHAPES])
def test_tensorwise_rows_every_launch_shape(s, h, label):
    inp = random_case(270 + s % 97 + h % 89, s, h, 64, 5, row_frac=0.5)
    X = inp["X"]
    say(f"  launch: tensor-wise rows {label} s={s} h={h}")
    mask, idx, n_out, idx_r = _gpu_detect(X, 6.0)
    Xq, c_x, X_O = i8.quantize_tensorwise(T(X), mask, idx, n_out)
    torch.cuda.synchronize()
    Xq_r, cx_r, XO_r = oracle.quantize_tensorwise(X, idx_r)
    assert np.array_equal(H(Xq), Xq_r), "tensor-wise Xq differs"
    assert np.array_equal(H(c_x).view(np.uint32), cx_r.view(np.uint32)), "tensor-wise c_x differs"
    _check_XO(X_O, XO_r)


@pytest.mark.parametrize("seed,s,h,o,nout,alpha", SHAPES, ids=IDS)
def test_one_call_variant_forwards(seed, s, h, o, nout, alpha):
    """forward_tensorwise / forward_zeropoint (detection accumulated in the
    workspace, the quantiser writing the index list) give the separate calls'
    C bit for bit, and the oracle's within the bar."""
    inp = random_case(280 + seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"].copy(), inp["W"]
    X[: s // 2] += np.float16(0.75)                    # shifted rows for the zero points
    b = (np.random.default_rng(seed).standard_normal(o) * 0.5).astype(np.float16) if seed % 2 else None
    Xd, Wd = T(X), T(W)
    bd = T(b) if b is not None else None
    say(f"  launch: one-call tensor-wise / zeropoint s={s} h={h} o={o} |O|={nout} alpha={alpha}")
    wt = i8.quantize_weights(Wd, "tensor")
    wz = i8.quantize_weights(Wd, "zeropoint")
    Ct = i8.forward_tensorwise(Xd, wt[0], wt[1], Wd, alpha, bias=bd)
    Cz = i8.forward_zeropoint(Xd, wz, Wd, alpha, bias=bd)
    Ct_sep = i8.variant_forward(Xd, wt, Wd, "tensor", alpha, bias=bd)
    Cz_sep = i8.variant_forward(Xd, wz, Wd, "zeropoint", alpha, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(Ct, Ct_sep), "one-call tensor-wise forward differs from the separate calls"
    assert torch.equal(Cz, Cz_sep), "one-call zeropoint forward differs from the separate calls"
    check_C(Ct, oracle.variant_forward(X, W, "tensor", alpha, bias=b))
    check_C(Cz, oracle.variant_forward(X, W, "zeropoint", alpha, bias=b))


def test_one_call_forwards_share_a_workspace():
    """One workspace, sized for the largest zeropoint case, serves every
    one-call forward in turn (absmax, tensor-wise, zeropoint, the
    inline-quantisation and the single-launch decode forwards), across
    shapes and both prologue paths (the accumulator must come back to zero
    after each)."""
    seq = [("zeropoint", 300, 640, 320), ("vector", 8, 1024, 256), ("tensor", 40, 512, 192),
           ("inline", 150, 1024, 256), ("zeropoint", 5, 1024, 128), ("decode", 12, 640, 192),
           ("vector", 260, 640, 576), ("tensor", 3, 192, 64), ("inline", 300, 192, 320),
           ("zeropoint", 17, 192, 320)]
    ws = i8.forward_workspace(300, 1024, DEV, zeropoint=True)
    for k, (scheme, s, h, o) in enumerate(seq):
        inp = random_case(300 + k, s, h, o, 3, row_frac=0.5)
        Xd, Wd = T(inp["X"]), T(inp["W"])
        say(f"  launch: shared workspace {scheme} s={s} h={h} o={o}")
        qw = i8.quantize_weights(Wd, scheme if scheme in ("zeropoint", "tensor") else "vector")
        if scheme == "zeropoint":
            C = i8.forward_zeropoint(Xd, qw, Wd, workspace=ws)
        elif scheme == "tensor":
            C = i8.forward_tensorwise(Xd, qw[0], qw[1], Wd, workspace=ws)
        elif scheme == "inline":
            C = i8.forward_inline_quant(Xd, qw[0], qw[1], Wd, workspace=ws)
        elif scheme == "decode":
            C = i8.forward_decode(Xd, qw[0], qw[1], Wd, workspace=ws)
        else:
            C = i8.forward(Xd, qw[0], qw[1], Wd, workspace=ws)
        C_sep = i8.variant_forward(Xd, qw, Wd, scheme if scheme in ("zeropoint", "tensor") else "vector")
        torch.cuda.synchronize()
        assert torch.equal(C, C_sep), f"{scheme} call {k} differs from the separate calls"
    acc = H(ws[: i8.ACC_BYTES])
    assert not acc.any(), "the accumulator is not zero after the calls"
