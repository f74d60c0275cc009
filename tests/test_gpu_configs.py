"""GPU parity at the full sizes of every workload, in the launch configuration
the benchmark times (i8mm_forward after the load-time weight conversion),
compared with the oracle over every element.

Bit-exact over the whole input and output: the outlier set, Xq, c_x, X_O,
the converted weights Wq (as W_i8 transposed) and c_w of every column, and
the int32 accumulator C_i32 of every output element (i8mm_int8_gemm_i32 runs
the product kernel's main loop). C is compared with the oracle's C over
every output element, within 2e-3 ||C_ref||_inf. On top of that, every
output element must lie inside the closed-form error bound
|C - X W| <= sum_k (|w| m_i + |x| m'_j + m_i m'_j / 254) / 254 (from the
absmax/254 per-element bound), with X W taken in fp32 on the GPU.

The oracle's work is spread over column chunks and threads (columns are
independent), which changes none of its arithmetic.
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_detect, check_rows, oracle_weights_by_columns, say
from workloads import CONFIGS, get_config, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "opt67b_ffn1_prefill", "b175_ffn1_decode", "b175_qkv_prefill"] + \
        [n for n in CONFIGS if n.startswith("sweep_")]

COL_CHUNK = 4096


def _bound_check(Xd, Wd, C, idx_r):
    s, h = Xd.shape
    keep = torch.ones(h, dtype=torch.bool, device=DEV)
    if idx_r.size:
        keep[torch.from_numpy(idx_r.astype(np.int64)).to(DEV)] = False
    X32 = Xd.float()
    W32 = Wd.float()
    Xa = X32.abs() * keep[None, :]
    m = Xa.max(dim=1).values
    Wa = W32.abs()
    mw = Wa.max(dim=0).values
    nk = float(keep.sum().item())
    Wk = Wa * keep[:, None]
    bound = (m[:, None] * Wk.sum(dim=0)[None, :] + Xa.sum(dim=1)[:, None] * mw[None, :]
             + nk * m[:, None] * mw[None, :] / 254.0) / 254.0
    ref = X32 @ W32
    fp32_err = h * 2.0 ** -23 * (X32.abs() @ Wa)
    Cf = C.float()
    ulp = torch.where(Cf.abs() < 2 ** -14, torch.full_like(Cf, 2.0 ** -24),
                      2.0 ** (torch.floor(torch.log2(Cf.abs().clamp_min(2 ** -14))) - 10))
    viol = ((Cf - ref).abs() > bound * (1 + 1e-4) + 0.5 * ulp + fp32_err + 1e-6).sum().item()
    assert viol == 0, f"{viol} outputs outside the closed-form error bound"


@pytest.mark.parametrize("name", NAMES)
def test_full_size_config(name):
    w = get_config(name)
    s, h, o = w.s, w.h, w.o
    say(f"[{name}] generating s={s} h={h} o={o}")
    inp = make_inputs(w)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    say(f"[{name}] launch: quantize_colwise_weights + forward + int8_gemm_i32")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(Xd, Wq, c_w, Wd, w.alpha, workspace=ws)
    v = i8.forward_workspace_views(ws, s, h)
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    torch.cuda.synchronize()

    say(f"[{name}] checking detection and row quantisation (every element)")
    idx_r = check_detect(X, w.alpha, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == sorted(inp["planted"].tolist())
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])

    say(f"[{name}] checking the weight conversion (every column)")
    Wq_t_r, cw_r = oracle_weights_by_columns(W)
    Wq_rows = i8.panels_to_rows(Wq)
    for j0 in range(0, o, COL_CHUNK):
        j1 = min(o, j0 + COL_CHUNK)
        assert np.array_equal(H(Wq_rows[j0:j1]), Wq_t_r[j0:j1]), f"Wq differs in columns {j0}..{j1 - 1}"
    del Wq_rows
    assert np.array_equal(H(c_w).view(np.uint32), cw_r.view(np.uint32)), "c_w differs"

    say(f"[{name}] checking C_i32 (every element) and C (every element, 2e-3)")
    Ci_r = oracle.int8_matmul_i32(Xq_r, Wq_t_r)
    err, norm = 0.0, 0.0
    for j0 in range(0, o, COL_CHUNK):
        j1 = min(o, j0 + COL_CHUNK)
        Ci_g = H(Ci[:, j0:j1])
        bad = np.argwhere(Ci_g != Ci_r[:, j0:j1])
        assert bad.size == 0, f"C_i32 differs at {(bad[:5] + [0, j0]).tolist()}"
        CO = oracle.outlier_matmul(XO_r, W[:, j0:j1], idx_r)
        R = oracle.dequantize_and_add(Ci_r[:, j0:j1], cx_r, cw_r[j0:j1], CO).astype(np.float64)
        G = H(C[:, j0:j1]).astype(np.float64)
        assert np.isfinite(G).all() and np.isfinite(R).all()
        err = max(err, float(np.abs(G - R).max()))
        norm = max(norm, float(np.abs(R).max()))
    del Ci, Ci_r
    assert err <= 2e-3 * norm, f"max |C - C_ref| = {err:.3e} > 2e-3 * {norm:.3e}"
    say(f"[{name}] max |C - C_ref| / ||C_ref|| = {err / norm:.2e} over all {s * o} outputs")
    _bound_check(Xd, Wd, C, idx_r)
