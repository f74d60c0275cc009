"""The single-launch decode forward (i8mm_forward_decode, s <= 16) against
the oracle: the outlier set, Xq, c_x and X_O bit for bit, C within 2e-3
||C_ref||_inf ([DIGEST] "The Full LLM.int8() Algorithm", Steps 1-5), and
C bit for bit equal to the three-launch forward's on the same inputs (the
same codes, constants, int32 products and epilogue arithmetic)."""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, check_rows, say
from workloads import get_config, make_inputs, random_case

pytestmark = pytest.mark.gpu

# (seed, s, h, o, planted outlier columns, alpha)
SHAPES = [(1, 1, 256, 64, 2, 6.0), (2, 3, 1024, 256, 5, 6.0), (3, 8, 4096, 512, 7, 6.0),
          (4, 16, 2048, 384, 3, 6.0), (5, 9, 12288, 1024, 7, 6.0), (6, 16, 1024, 128, 40, 6.0),
          (7, 5, 640, 192, 0, 6.0), (8, 4, 256, 64, 3, 0.0), (9, 12, 512, 256, 6, float("inf")),
          (10, 2, 64, 64, 1, 6.0)]


def _both(X, W, alpha, fp16_weights=True, bias=None):
    s, h = X.shape
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    bd = None if bias is None else T(bias)
    Wp = Wd if fp16_weights else None
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward_decode(Xd, Wq, c_w, Wp, alpha, workspace=ws, bias=bd)
    C3 = i8.forward(Xd, Wq, c_w, Wp, alpha, bias=bd)
    torch.cuda.synchronize()
    return C, C3, ws


@pytest.mark.parametrize("seed,s,h,o,nout,alpha", SHAPES, ids=[f"s{c[1]}h{c[2]}o{c[3]}n{c[4]}a{c[5]}" for c in SHAPES])
def test_single_launch_decode(seed, s, h, o, nout, alpha):
    inp = random_case(800 + seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    say(f"  launch: forward_decode s={s} h={h} o={o} alpha={alpha}")
    C, C3, ws = _both(X, W, alpha)
    v = i8.forward_workspace_views(ws, s, h)
    idx_r = check_detect(X, alpha, v["mask"], v["idx"], v["n_out"])
    check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    check_C(C, oracle.forward(X, W, alpha)["C"])
    assert torch.equal(C, C3), "single-launch C differs from the three-launch forward's"


@pytest.mark.parametrize("s", [1, 8])
def test_single_launch_decode_without_fp16_weights_and_with_bias(s):
    h, o = 2048, 256
    inp = random_case(860 + s, s, h, o, 6, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    b = ((np.arange(o) % 5 - 2) * 0.25).astype(np.float16)
    say(f"  launch: forward_decode s={s} without fp16 W, with bias")
    C, C3, _ = _both(X, W, 6.0, fp16_weights=False, bias=b)
    check_C(C, oracle.forward(X, W, 6.0, fp16_weights=False, bias=b)["C"])
    assert torch.equal(C, C3)


def test_single_launch_decode_full_size():
    """The 175B-style FFN expansion decode layer (8 x 12288 x 49152) over
    every output element."""
    w = get_config("b175_ffn1_decode")
    inp = make_inputs(w)
    X, W = inp["X"], inp["W"]
    say(f"  launch: forward_decode s={w.s} h={w.h} o={w.o}")
    C, C3, ws = _both(X, W, w.alpha)
    v = i8.forward_workspace_views(ws, w.s, w.h)
    idx_r = check_detect(X, w.alpha, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == sorted(inp["planted"].tolist())
    check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    rel = check_C(C, oracle.forward(X, W, w.alpha)["C"])
    assert torch.equal(C, C3)
    say(f"  max |C - C_ref| / ||C_ref|| = {rel:.2e}")
