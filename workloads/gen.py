"""Seeded synthetic activations X and weights W shaped like the pages' layers.

Page tags used in this file:
  [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale"
           (paper-graph-ui.vercel.app digest of arXiv 2208.07339)
  [PY]     "LLM.int8() 完全拆解：系统离群值的涌现与混合精度分解" (pinghaoyang.com.cn)

What the inputs imitate (shapes and statistics only; no model weights or
activations are used or needed):
  * hidden states X [s, h] are roughly N(0, 1) with a handful of outlier
    feature columns, "at most 7" for models up to 13B, that carry large
    one-sided magnitudes in most sequence positions ([DIGEST] "Outlier Feature
    Detection and Characterization", bullets Sparsity / Systematicity /
    Asymmetry; [PY] "核心发现").
  * weights W [h, o] are N(0, 0.02), std 0.02, generated in fp32 then cast to
    fp16.

Conventions (the pages leave these open):
  * numpy ``default_rng(seed)`` (PCG64), a fresh generator per tensor set.
  * draw order: base X, outlier columns, per-column signs, per-column row sets,
    magnitudes, then W.
  * base X redraws any |x| >= 5.5 so that the outlier set is exactly the
    planted set (otherwise a 4096x12288 draw has a few-percent chance of a
    natural |x| >= 6 element, which would break the |O| = 0 sweep point).
  * one random sign per outlier column (one-sided outliers).
  * each outlier column gets exactly round(frac * s) rows, without replacement.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "SWEEP_POINTS",
    "get_config",
    "make_X",
    "make_W",
    "make_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and outlier recipe of one synthetic linear layer C = X W."""

    name: str
    s: int                      # rows of X (sequence positions)
    h: int                      # hidden size (reduction dimension)
    o: int                      # output features
    n_outliers: int             # number of planted outlier columns
    row_frac: float             # fraction of rows carrying the outlier value
    mag_lo: float = 6.0         # outlier magnitude ~ U(mag_lo, mag_hi)
    mag_hi: float = 20.0
    fixed_cols: Optional[Tuple[int, ...]] = None  # planted columns, else random
    w_std: float = 0.02
    alpha: float = 6.0
    seed: int = 0
    decode: bool = False        # weight-streaming (bandwidth-bound) shape

    @property
    def int_ops(self) -> int:
        """Dense-equivalent operation count 2*s*h*o."""
        return 2 * self.s * self.h * self.o


def _sweep() -> List[Workload]:
    pts = [Workload("sweep_o0", 4096, 8192, 28672, 0, 0.0)]
    for n in (7, 64):
        for f in (0.06, 0.28, 0.75, 1.0):
            pts.append(Workload(f"sweep_o{n}_r{int(round(f * 100))}", 4096, 8192, 28672, n, f))
    return pts


CONFIGS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 16, 256, 512, 2, 0.3, mag_lo=8.0, mag_hi=20.0, fixed_cols=(3, 100)),
    "opt67b_ffn1_prefill": Workload("opt67b_ffn1_prefill", 2048, 4096, 16384, 6, 0.75),
    "b175_ffn1_decode": Workload("b175_ffn1_decode", 8, 12288, 49152, 7, 1.0, decode=True),
    "b175_qkv_prefill": Workload("b175_qkv_prefill", 4096, 12288, 36864, 7, 0.75),
}
SWEEP_POINTS: List[Workload] = _sweep()
for _w in SWEEP_POINTS:
    CONFIGS[_w.name] = _w


def get_config(name: str) -> Workload:
    return CONFIGS[name]


def _base_normal(rng: np.random.Generator, shape: Tuple[int, int], clip: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    bad = np.abs(x) >= clip
    while bad.any():
        x[bad] = rng.standard_normal(int(bad.sum()), dtype=np.float32)
        bad = np.abs(x) >= clip
    return x


def make_X(w: Workload, rng: Optional[np.random.Generator] = None,
           s: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Return (X fp16 [s, h], planted outlier columns int64 ascending)."""
    if rng is None:
        rng = np.random.default_rng(w.seed)
    s = w.s if s is None else s
    h = w.h
    x = _base_normal(rng, (s, h), 5.5)
    if w.fixed_cols is not None:
        cols = np.array(w.fixed_cols, dtype=np.int64)
    else:
        cols = np.sort(rng.choice(h, size=w.n_outliers, replace=False)).astype(np.int64)
    signs = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=len(cols))
    nrows = int(round(w.row_frac * s))
    rowsets = [rng.choice(s, size=nrows, replace=False) for _ in cols]
    for c, sg, rows in zip(cols, signs, rowsets):
        mags = rng.uniform(w.mag_lo, w.mag_hi, size=nrows).astype(np.float32)
        x[rows, c] = sg * mags
    return x.astype(np.float16), cols


def make_W(w: Workload, rng: Optional[np.random.Generator] = None,
           chunk_rows: int = 1024) -> np.ndarray:
    """Return W fp16 [h, o] ~ N(0, w_std), drawn row-chunk by row-chunk."""
    if rng is None:
        rng = np.random.default_rng(w.seed)
    out = np.empty((w.h, w.o), dtype=np.float16)
    for r0 in range(0, w.h, chunk_rows):
        r1 = min(w.h, r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0, w.o), dtype=np.float32)
        blk *= np.float32(w.w_std)
        out[r0:r1] = blk.astype(np.float16)
    return out


def make_inputs(w: Workload, with_W: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one workload from one fresh generator: X, planted cols, W."""
    rng = np.random.default_rng(w.seed)
    X, cols = make_X(w, rng)
    out = {"X": X, "planted": cols}
    if with_W:
        out["W"] = make_W(w, rng)
    return out


def random_case(seed: int, s: int, h: int, o: int, n_outliers: int,
                row_frac: float = 0.5, alpha: float = 6.0) -> Dict[str, np.ndarray]:
    """Small random case for property/parity tests (any shape)."""
    w = Workload(f"rand{seed}", s, h, o, n_outliers, row_frac, seed=seed, alpha=alpha)
    return make_inputs(w)


def planted_on_row_subset(X: np.ndarray, cols: Sequence[int], rows: Sequence[int],
                          value: float) -> np.ndarray:
    """Return a copy of X with X[rows, cols] = value (fp16)."""
    Y = X.copy()
    for c in cols:
        Y[np.asarray(rows, dtype=np.int64), c] = np.float16(value)
    return Y
