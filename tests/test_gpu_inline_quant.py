"""The forward with the row quantisation folded into the product
(i8mm_forward_inline_quant: the int8 codes of X made inside the product
kernel while it stages its operand tiles, never stored) against the oracle:
the outlier set, c_x and X_O bit for bit, C within 2e-3 ||C_ref||_inf
([DIGEST] "The Full LLM.int8() Algorithm", Steps 1-5), and C bit for bit
equal to i8mm_forward's on the same inputs (the same codes from the same
rounding, the same int32 products and epilogue). The shapes cover ragged
row and column tiles, reduction lengths ending in half a 128-column stage,
outlier columns on the 16-column chunk and 128-column stage boundaries, zero
rows, alpha = 0 and +inf, the largest h, and the full-size prefill layers.
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, say
from workloads import get_config, make_inputs, planted_on_row_subset, random_case

pytestmark = pytest.mark.gpu

# (seed, s, h, o, planted outlier columns, alpha)
SHAPES = [(1, 129, 256, 512, 2, 6.0), (2, 300, 640, 576, 5, 6.0), (3, 513, 384, 768, 40, 6.0),
          (4, 257, 1088, 832, 3, 6.0), (5, 160, 192, 320, 1, 6.0), (6, 130, 4096, 256, 7, 6.0),
          (7, 200, 512, 256, 0, 6.0), (8, 144, 256, 128, 3, 0.0), (9, 150, 512, 384, 6, float("inf")),
          (10, 129, 133120, 256, 4, 6.0)]


def _run(X, W, alpha, fp16_weights=True, bias=None):
    s, h = X.shape
    Xd, Wd = T(X), T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    bd = None if bias is None else T(bias)
    Wp = Wd if fp16_weights else None
    ws = i8.forward_workspace(s, h, DEV)
    ws.fill_(0x5A)
    ws[:i8.ACC_BYTES].zero_()
    C = i8.forward_inline_quant(Xd, Wq, c_w, Wp, alpha, workspace=ws, bias=bd)
    C2 = i8.forward(Xd, Wq, c_w, Wp, alpha, bias=bd)
    torch.cuda.synchronize()
    return C, C2, ws


def _check_intermediates(X, alpha, ws):
    s, h = X.shape
    v = i8.forward_workspace_views(ws, s, h)
    idx_r = check_detect(X, alpha, v["mask"], v["idx"], v["n_out"])
    _, cx_r, XO_r = oracle.quantize_rowwise(X, idx_r)
    assert np.array_equal(H(v["c_x"]).view(np.uint32), cx_r.view(np.uint32)), "c_x differs"
    n = idx_r.size
    XO = H(v["X_O"])
    assert np.array_equal(XO[:, :n].view(np.uint16), XO_r.view(np.uint16)), "X_O differs"
    assert not XO[:, n:(n + 31) // 32 * 32].view(np.uint16).any(), "X_O padding not zero"
    assert bool((v["Xq"].view(torch.uint8) == 0x5A).all()), "the Xq region was written"
    assert not H(ws[:i8.ACC_BYTES]).any(), "accumulator not left zero"
    return idx_r


@pytest.mark.parametrize("seed,s,h,o,nout,alpha", SHAPES, ids=[f"s{c[1]}h{c[2]}o{c[3]}n{c[4]}a{c[5]}" for c in SHAPES])
def test_inline_quant_forward(seed, s, h, o, nout, alpha):
    inp = random_case(900 + seed, s, h, o, nout, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    say(f"  launch: forward_inline_quant s={s} h={h} o={o} alpha={alpha}")
    C, C2, ws = _run(X, W, alpha)
    _check_intermediates(X, alpha, ws)
    check_C(C, oracle.forward(X, W, alpha)["C"])
    assert torch.equal(C, C2), "C differs from the two-pass forward's"


def test_inline_quant_outliers_on_chunk_and_stage_boundaries():
    """Outlier columns at the first and last column of 16-column chunks and
    128-column stages, and the last column of a half stage; zero rows."""
    s, h, o = 333, 448, 320
    inp = random_case(950, s, h, o, 0, row_frac=0.5)
    cols = [0, 15, 16, 127, 128, 255, 256, 383, 384, h - 1]
    X = planted_on_row_subset(inp["X"], cols, list(range(0, s, 3)), -9.5)
    X[[5, 77, 300]] = 0
    say(f"  launch: forward_inline_quant s={s} h={h} o={o}, outliers {cols}")
    C, C2, ws = _run(X, inp["W"], 6.0)
    assert _check_intermediates(X, 6.0, ws).tolist() == cols
    check_C(C, oracle.forward(X, inp["W"], 6.0)["C"])
    assert torch.equal(C, C2)


def test_inline_quant_without_fp16_weights_and_with_bias():
    s, h, o = 300, 1024, 512
    inp = random_case(960, s, h, o, 6, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    b = ((np.arange(o) % 5 - 2) * 0.25).astype(np.float16)
    say("  launch: forward_inline_quant without fp16 W, with bias")
    C, C2, _ = _run(X, W, 6.0, fp16_weights=False, bias=b)
    check_C(C, oracle.forward(X, W, 6.0, fp16_weights=False, bias=b)["C"])
    assert torch.equal(C, C2)


def test_inline_quant_rejects_few_rows():
    X = torch.zeros((i8.INLINE_QUANT_MIN_ROWS - 1, 256), dtype=torch.float16, device=DEV)
    Wq, c_w = i8.quantize_colwise_weights(torch.zeros((256, 64), dtype=torch.float16, device=DEV))
    with pytest.raises(i8.I8MMError):
        i8.forward_inline_quant(X, Wq, c_w, None, 6.0)


@pytest.mark.parametrize("name", ["opt67b_ffn1_prefill", "b175_qkv_prefill"])
def test_inline_quant_full_size(name):
    """Every output element of the full-size prefill layers equals the
    two-pass forward's, bit for bit."""
    w = get_config(name)
    inp = make_inputs(w)
    X, W = inp["X"], inp["W"]
    say(f"  launch: forward_inline_quant s={w.s} h={w.h} o={w.o}")
    C, C2, ws = _run(X, W, w.alpha)
    idx_r = _check_intermediates(X, w.alpha, ws)
    assert idx_r.tolist() == sorted(inp["planted"].tolist())
    same = C.view(torch.int16) == C2.view(torch.int16)
    assert bool(same.all()), f"{int((~same).sum())} of {C.numel()} outputs differ from the two-pass forward's"
