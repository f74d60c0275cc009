"""The forward's prologue for few rows, against the oracle: up to 8 rows and
24 KiB of X it runs in one launch (every block scans all of X for the mask
and the row maxima, then quantises its own 128-column slab), above that in
two (the slab pair). The shapes sit on both sides of that size, at one
slab, at a half-filled last slab and at the narrowest width. Every case
checks bit for bit the outlier set, Xq, c_x and X_O with its zero padding,
and C_i32; C within 2e-3 ||C_ref||_inf ([DIGEST] "The Full LLM.int8()
Algorithm", Steps 1-5)."""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, check_rows, say
from workloads import random_case

pytestmark = pytest.mark.gpu

# (s, h): 2 s h bytes of X against the 24 KiB limit
ONE_LAUNCH = [(1, 64), (8, 64), (1, 256), (3, 1216), (4, 2112), (2, 4096), (3, 4096), (8, 1536), (1, 12288)]
TWO_LAUNCH = [(8, 1600), (3, 4160), (1, 12352), (2, 6208), (8, 12288)]
SHAPES = [(s, h, "one launch") for s, h in ONE_LAUNCH] + [(s, h, "slab pair") for s, h in TWO_LAUNCH]
IDS = [f"s{s}h{h}-{'one' if lab == 'one launch' else 'pair'}" for s, h, lab in SHAPES]


def _run(X, W, alpha, ws=None):
    s, h = X.shape
    Wd = T(W)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    if ws is None:
        ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(T(X), Wq, c_w, Wd, alpha, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    torch.cuda.synchronize()
    idx_r = check_detect(X, alpha, v["mask"], v["idx"], v["n_out"])
    Xq_r, _, _ = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])
    Wq_t_r, _ = oracle.quantize_colwise_weights(W)
    bad = np.argwhere(H(Ci) != oracle.int8_matmul_i32(Xq_r, Wq_t_r))
    assert bad.size == 0, f"C_i32 differs at {bad[:5].tolist()}"
    check_C(C, oracle.forward(X, W, alpha)["C"])
    return idx_r


def _edges(X):
    """Outliers in the first and the last column (one row each), a zero row."""
    s, h = X.shape
    X = X.copy()
    X[0, 0] = 7.5
    X[s - 1, h - 1] = -9.0
    if s > 2:
        X[1, :] = 0
    return X


@pytest.mark.parametrize("s,h,route", SHAPES, ids=IDS)
def test_few_rows(s, h, route):
    o = 192
    inp = random_case(2100 + s * 7 + h, s, h, o, min(5, h // 16), row_frac=0.5)
    X, W = _edges(inp["X"]), inp["W"]
    say(f"  launch: forward ({route}) s={s} h={h} o={o}")
    idx_r = _run(X, W, 6.0)
    assert idx_r[0] == 0 and idx_r[-1] == h - 1


@pytest.mark.parametrize("s,h", [(8, 1536), (1, 64), (8, 1600)], ids=["one-8x1536", "one-1x64", "pair-8x1600"])
def test_every_column_an_outlier(s, h):
    """alpha = 0: every column is in O, X_O is all of X, the codes are all
    zero and c_x is 1 (the pages' zero-row convention)."""
    o = 64
    inp = random_case(2200 + s + h, s, h, o, 0)
    say(f"  launch: forward alpha=0 s={s} h={h}")
    idx_r = _run(inp["X"], inp["W"], 0.0)
    assert idx_r.size == h


@pytest.mark.parametrize("s,h", [(4, 2112), (8, 1600)], ids=["one-4x2112", "pair-8x1600"])
def test_no_outliers(s, h):
    o = 64
    inp = random_case(2300 + s + h, s, h, o, 3)
    say(f"  launch: forward alpha=inf s={s} h={h}")
    idx_r = _run(inp["X"], inp["W"], float("inf"))
    assert idx_r.size == 0


@pytest.mark.parametrize("s,h", [(8, 1536), (8, 1600)], ids=["one-8x1536", "pair-8x1600"])
def test_nan_beside_an_outlier(s, h):
    """A column holding a NaN and an element at alpha is in O; a NaN alone
    does not reach alpha. Only the outlier set is defined for such input."""
    o = 64
    inp = random_case(2400 + s + h, s, h, o, 0)
    X = inp["X"].copy()
    X[0, 3] = np.nan
    X[s - 1, 3] = 10.0
    X[1, 7] = np.nan
    X[2, h - 65] = -6.0
    say(f"  launch: forward with NaN s={s} h={h}")
    Wd = T(inp["W"])
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    i8.forward(T(X), Wq, c_w, Wd, 6.0, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    torch.cuda.synchronize()
    idx_r = check_detect(X, 6.0, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == [3, h - 65]


def test_routes_share_a_workspace():
    """One workspace, sized for the largest case, through both few-row routes
    and the many-row one in turn: each leaves the workspace as the next one
    needs it (the one-launch route uses no accumulator at all)."""
    cases = [(8, 1536), (8, 1600), (16, 1024), (1, 64), (8, 1600), (4, 2112)]
    smax = max(c[0] for c in cases)
    hmax = max(c[1] for c in cases)
    ws = i8.forward_workspace(smax, hmax, DEV)
    for k, (s, h) in enumerate(cases):
        inp = random_case(2500 + k, s, h, 128, 4, row_frac=0.5)
        say(f"  launch: forward in a shared workspace s={s} h={h}")
        _run(_edges(inp["X"]), inp["W"], 6.0, ws=ws)
