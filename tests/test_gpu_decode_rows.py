"""The products at each row-count boundary, against the oracle: the K-split
weight-streaming kernel up to 16 rows (narrow layers, and layers its blocks
fill evenly), the column-split one with X's codes in LDS otherwise up to
128 rows (1, 2, 3, 4, 6 or 8 row groups of 16), the tiled product above
128. Checked bit for bit: the outlier set, Xq, c_x, X_O and C_i32; C
within 2e-3 ||C_ref||_inf. The one-call forward, the four-step product and
the int32 product all dispatch on s the same way. The column-split kernel
stages K in chunks of four 64-wide steps, two chunks per loop: the uneven
shapes give an odd number of chunks, a last chunk with one to three steps,
a single step, and column counts that are not a multiple of 256."""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, check_rows, say
from workloads import random_case

pytestmark = pytest.mark.gpu

ROWS = [16, 17, 32, 33, 48, 49, 64, 65, 96, 97, 128, 129]
UNEVEN = [(40, 4160, 192, 5), (24, 64, 64, 1), (64, 448, 320, 3), (17, 192, 128, 2), (56, 1216, 576, 9),
          (100, 704, 192, 4), (128, 64, 3136, 2)]
# Few rows on wide layers that the K-split kernel would not fill evenly: the
# forward picks the column-split kernel with one row group from the column
# count (on 256 CUs); the test checks parity only.
WIDE_FEW = [(1, 256, 36864, 2), (8, 320, 28672, 3), (16, 192, 16384, 1), (9, 128, 17408, 4)]


def _check_shape(seed, s, h, o, nout):
    inp = random_case(seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    say(f"  launch: forward + int8_gemm_i32 + int8_mixed_matmul s={s} h={h} o={o}")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    C4 = i8.int8_mixed_matmul(v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w, Wd)
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, v["mask"], v["idx"], v["n_out"])
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    Wq_t_r, cw_r = oracle.quantize_colwise_weights(W)
    Ci_r = oracle.int8_matmul_i32(Xq_r, Wq_t_r)
    bad = np.argwhere(H(Ci) != Ci_r)
    assert bad.size == 0, f"C_i32 differs at {bad[:5].tolist()}"
    check_C(C, oracle.forward(X, W, 6.0)["C"])
    assert torch.equal(C, C4), "the one-call forward and the four-step product differ"


@pytest.mark.parametrize("s", ROWS)
def test_row_group_boundaries(s):
    _check_shape(1700 + s, s, 4096, 1024, 6)


@pytest.mark.parametrize("s,h,o,nout", UNEVEN, ids=[f"s{c[0]}h{c[1]}o{c[2]}" for c in UNEVEN])
def test_uneven_k_and_columns(s, h, o, nout):
    _check_shape(1800 + s + h, s, h, o, nout)


@pytest.mark.parametrize("s,h,o,nout", WIDE_FEW, ids=[f"s{c[0]}h{c[1]}o{c[2]}" for c in WIDE_FEW])
def test_few_rows_on_wide_layers(s, h, o, nout):
    _check_shape(1900 + s + h, s, h, o, nout)


@pytest.mark.parametrize("s", [20, 40, 60, 90, 120])
def test_row_groups_without_fp16_weights_and_with_bias(s):
    h, o = 2048, 512
    inp = random_case(1760 + s, s, h, o, 5, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    b = ((np.arange(o) % 7 - 3) * 0.125).astype(np.float16)
    Xd, Wd = T(X), T(W)
    say(f"  launch: forward without fp16 W, with bias, s={s}")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    C = i8.forward(Xd, Wq, c_w, None, 6.0, bias=T(b))
    torch.cuda.synchronize()
    check_C(C, oracle.forward(X, W, 6.0, fp16_weights=False, bias=b)["C"])
