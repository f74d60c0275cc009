"""Parity at the size limits: the largest weight extent the products accept
(h * o just below 2^31: Wq and the fp16 weight rows are read through 32-bit
buffer offsets), on the two weight-streaming products (s <= 16, 17..64)
and the tiled one (s > 128), through the one-call forward the benchmark
times; and tall inputs
(up to 2^18 rows).

Every code of the converted weights, every c_w and every element of C_i32 is
compared bit for bit with the oracle, and every element of C within
2e-3 ||C_ref||_inf. W is the deterministic pattern
W[k, j] = ((7 k + 13 j) mod 251 - 125) / 64 (exact in fp16, every column
reaching the same absmax), so that making 2^31 weights stays quick; X is
seeded N(0, 1) with planted outlier columns.

The fp16 W spans 4 GiB here, more than 2^31 bytes: the test then plants +inf
in a row of W outside O, at the element an offset of 2^31 bytes from the
first tile's columns would reach, and requires C to stay bit-identical (the
product reads only the rows W[idx, :]; lanes with no outlier row to stage
must read nothing).
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_detect, check_rows, oracle_weights_by_columns, say
from workloads import random_case

pytestmark = pytest.mark.gpu

H_MAX_EXTENT, O_MAX_EXTENT = 32768, 65472          # h * o = 2 145 386 496 < 2^31
COL_CHUNK = 4096


def _pattern_weights(h, o):
    vals = (np.arange(251) - 125).astype(np.float16) * np.float16(1.0 / 64)
    jj = (np.arange(o, dtype=np.int64) * 13) % 251
    rows = vals[(np.arange(251)[:, None] + jj[None, :]) % 251]   # rows[m, j] = vals[(m + 13 j) mod 251]
    return rows[(np.arange(h) * 7) % 251]


@pytest.fixture(scope="module")
def max_extent_weights():
    h, o = H_MAX_EXTENT, O_MAX_EXTENT
    assert h * o < 2 ** 31 and 2 * h * o > 2 ** 31
    say(f"  generating W {h}x{o} and its oracle conversion")
    W = _pattern_weights(h, o)
    Wq_t_r, cw_r = oracle_weights_by_columns(W)
    Wd = T(W)
    say("  launch: quantize_colwise_weights at the largest extent")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    torch.cuda.synchronize()
    rows = i8.panels_to_rows(Wq)
    for j0 in range(0, o, COL_CHUNK):
        assert np.array_equal(H(rows[j0:j0 + COL_CHUNK]), Wq_t_r[j0:j0 + COL_CHUNK]), f"Wq differs in columns {j0}.."
    del rows
    assert np.array_equal(H(c_w).view(np.uint32), cw_r.view(np.uint32)), "c_w differs"
    yield W, Wd, Wq, c_w, Wq_t_r, cw_r
    del Wd, Wq, c_w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("s", [16, 40, 300])
def test_largest_weight_extent(max_extent_weights, s):
    W, Wd, Wq, c_w, Wq_t_r, cw_r = max_extent_weights
    h, o = W.shape
    X = random_case(990 + s, s, h, 64, 5, row_frac=0.5)["X"]
    Xd = T(X)
    say(f"  launch: forward + int8_gemm_i32 s={s} h={h} o={o}")
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, v["mask"], v["idx"], v["n_out"])
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    Ci_r = oracle.int8_matmul_i32(Xq_r, Wq_t_r)
    bad = np.argwhere(H(Ci) != Ci_r)
    assert bad.size == 0, f"C_i32 differs at {bad[:5].tolist()}"
    err, norm = 0.0, 0.0
    for j0 in range(0, o, COL_CHUNK):
        j1 = min(o, j0 + COL_CHUNK)
        CO = oracle.outlier_matmul(XO_r, W[:, j0:j1], idx_r)
        R = oracle.dequantize_and_add(Ci_r[:, j0:j1], cx_r, cw_r[j0:j1], CO).astype(np.float64)
        G = H(C[:, j0:j1]).astype(np.float64)
        assert np.isfinite(G).all() and np.isfinite(R).all()
        err = max(err, float(np.abs(G - R).max()))
        norm = max(norm, float(np.abs(R).max()))
    assert err <= 2e-3 * norm, f"max |C - C_ref| = {err:.3e} > 2e-3 * {norm:.3e}"
    say(f"  max |C - C_ref| / ||C_ref|| = {err / norm:.2e}")

    if s <= 16:
        say(f"  launch: forward_decode s={s} at the largest extent")
        C1 = i8.forward_decode(Xd, Wq, c_w, Wd, 6.0, workspace=i8.forward_workspace(s, h, DEV))
        torch.cuda.synchronize()
        assert torch.equal(C1, C), "forward_decode differs from forward"

    # +inf in a row outside O, 2^31 bytes past the first column of W
    r_inf, c_inf = divmod(2 ** 30, o)
    assert r_inf not in idx_r.tolist() and idx_r.size % 16 != 0
    say(f"  launch: forward with W[{r_inf}, {c_inf}] = +inf (row outside O)")
    Wd[r_inf, c_inf] = float("inf")
    try:
        C2 = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
        torch.cuda.synchronize()
    finally:
        Wd[r_inf, c_inf] = float(W[r_inf, c_inf])
        torch.cuda.synchronize()
    same = (C2.view(torch.int16) == C.view(torch.int16))
    assert bool(same.all()), f"{int((~same).sum())} outputs changed by a W row outside O"


# Tall inputs: thousands of 256-row tiles against one or two weight tiles
# (the grouped tile order with fewer weight tiles than its group width),
# thousands of detection row blocks and a row-quantiser grid of 2^16 blocks.
TALL = [(2 ** 18, 64, 64, 1), (2 ** 18, 128, 320, 3), (100_001, 192, 256, 2)]


@pytest.mark.parametrize("s,h,o,nout", TALL, ids=[f"s{c[0]}h{c[1]}o{c[2]}" for c in TALL])
def test_tall_inputs(s, h, o, nout):
    inp = random_case(1200 + h, s, h, o, nout, row_frac=0.01)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    say(f"  launch: forward, forward_inline_quant, int8_gemm_i32 s={s} h={h} o={o}")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    C2 = i8.forward_inline_quant(Xd, Wq, c_w, Wd, 6.0)
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == sorted(inp["planted"].tolist())
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    Wq_t_r, cw_r = oracle_weights_by_columns(W)
    Ci_r = oracle.int8_matmul_i32(Xq_r, Wq_t_r)
    bad = np.argwhere(H(Ci) != Ci_r)
    assert bad.size == 0, f"C_i32 differs at {bad[:5].tolist()}"
    R = oracle.dequantize_and_add(Ci_r, cx_r, cw_r, oracle.outlier_matmul(XO_r, W, idx_r)).astype(np.float64)
    G = H(C).astype(np.float64)
    assert np.abs(G - R).max() <= 2e-3 * np.abs(R).max()
    assert torch.equal(C2, C), "forward_inline_quant differs from forward"
