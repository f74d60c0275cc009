"""GPU parity at the full sizes of every workload, in the launch configuration
the benchmark times (i8mm_forward after the load-time weight conversion).

Exact over the whole input: the outlier set, Xq, c_x and X_O. Exact on
sampled output columns (the conversion of each W column is independent):
Wq (as W_i8 transposed) and c_w. On sampled rows x columns: C_i32 exactly and C within
2e-3 ||C_ref||_inf of the oracle. Over every output element: the
closed-form error bound |C - X W| <= sum_k (|w| m_i + |x| m'_j + m_i m'_j / 254) / 254
(from the absmax/254 per-element bound), with X W taken in fp32 on the GPU.
"""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, check_detect, check_rows, say
from workloads import CONFIGS, get_config, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "opt67b_ffn1_prefill", "b175_ffn1_decode", "b175_qkv_prefill"] + \
        [n for n in CONFIGS if n.startswith("sweep_")]


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
    say(f"[{name}] launch: quantize_colwise_weights + forward")
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    ws = i8.forward_workspace(s, h, DEV)
    C = i8.forward(Xd, Wq, c_w, Wd, w.alpha, workspace=ws)
    torch.cuda.synchronize()
    v = i8.forward_workspace_views(ws, s, h)

    say(f"[{name}] checking intermediates")
    idx_r = check_detect(X, w.alpha, v["mask"], v["idx"], v["n_out"])
    assert idx_r.tolist() == sorted(inp["planted"].tolist())
    Xq_r, cx_r, XO_r = check_rows(X, idx_r, v["Xq"], v["c_x"], v["X_O"])

    rng = np.random.default_rng(123)
    cols = np.unique(np.concatenate([[0, o - 1], rng.choice(o, 254, replace=False)]))
    rows = np.unique(np.concatenate([[0, s - 1], rng.choice(s, min(s, 62), replace=False)]))
    cols_d = torch.from_numpy(cols).to(DEV)
    rows_d = torch.from_numpy(rows).to(DEV)
    Wq_s, cw_s = oracle.quantize_colwise_weights(W[:, cols])
    assert np.array_equal(H(i8.panels_to_rows(Wq.index_select(1, cols_d))), Wq_s), "Wq differs"
    assert np.array_equal(H(c_w.index_select(0, cols_d)).view(np.uint32), cw_s.view(np.uint32)), "c_w differs"

    say(f"[{name}] launch: int8_gemm_i32")
    Ci = i8.int8_gemm_i32(v["Xq"], Wq)
    torch.cuda.synchronize()
    Ci_s = H(Ci.index_select(0, rows_d).index_select(1, cols_d))
    del Ci
    assert np.array_equal(Ci_s, oracle.int8_matmul_i32(Xq_r[rows], Wq_s)), "C_i32 differs"
    C_ref = oracle.int8_mixed_matmul(Xq_r[rows], cx_r[rows], XO_r[rows], idx_r, Wq_s, cw_s, W[:, cols])
    rel = check_C(C.index_select(0, rows_d).index_select(1, cols_d), C_ref)
    say(f"[{name}] sampled max rel err {rel:.2e}")
    _bound_check(Xd, Wd, C, idx_r)
