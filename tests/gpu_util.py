"""Helpers shared by the GPU parity tests (host <-> device copies, checks)."""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def T(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def H(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def round_up(v: int, m: int) -> int:
    return (v + m - 1) // m * m


def check_detect(X: np.ndarray, alpha: float, mask_d, idx_d, n_d):
    mask_r, idx_r, n_r = oracle.outlier_columns(X, alpha)
    n = int(H(n_d)[0])
    assert n == n_r, f"|O| {n} != {n_r}"
    assert np.array_equal(H(mask_d).view(np.uint32), mask_r), "mask differs"
    assert np.array_equal(H(idx_d)[:n], idx_r), "idx differs"
    return idx_r


def check_rows(X: np.ndarray, idx_r: np.ndarray, Xq_d, cx_d, XO_d):
    Xq_r, cx_r, XO_r = oracle.quantize_rowwise(X, idx_r)
    Xq = H(Xq_d)
    bad = np.argwhere(Xq != Xq_r)
    assert bad.size == 0, f"Xq differs at {bad[:5].tolist()} ({Xq[tuple(bad[0])]} vs {Xq_r[tuple(bad[0])]})"
    assert np.array_equal(H(cx_d).view(np.uint32), cx_r.view(np.uint32)), "c_x differs"
    n = idx_r.size
    XO = H(XO_d)
    assert np.array_equal(XO[:, :n].view(np.uint16), XO_r.view(np.uint16)), "X_O differs"
    assert not XO[:, n:round_up(n, 32)].view(np.uint16).any(), "X_O padding not zero"
    return Xq_r, cx_r, XO_r


def check_C(C_d, C_ref: np.ndarray, tol: float = 2e-3):
    C = H(C_d).astype(np.float64)
    R = C_ref.astype(np.float64)
    assert np.isfinite(C).all() == np.isfinite(R).all()
    norm = np.abs(R).max() if R.size else 0.0
    err = np.abs(C - R).max() if R.size else 0.0
    assert err <= tol * norm + 1e-30, f"max |C - C_ref| = {err:.3e} > {tol} * {norm:.3e}"
    return err / norm if norm else 0.0


def host_threads() -> int:
    """Threads for host-side oracle work: the cores this process may run on,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_weights_by_columns(W: np.ndarray, chunk: int = 2048):
    """The oracle's load-time conversion of every column of W, evaluated on
    column chunks in parallel threads. Columns are converted independently
    (each has its own constant), so this is oracle.quantize_colwise_weights
    of the whole W; only the evaluation is spread over threads."""
    h, o = W.shape
    Wq_t = np.empty((o, h), np.int8)
    c_w = np.empty(o, np.float32)

    def job(j0):
        q, c = oracle.quantize_colwise_weights(W[:, j0:j0 + chunk])
        Wq_t[j0:j0 + chunk] = q
        c_w[j0:j0 + chunk] = c

    with ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(job, range(0, o, chunk)))
    return Wq_t, c_w
