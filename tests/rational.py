"""Exact rational brute force of LLM.int8() for tiny inputs (test helper).

Independent of ``oracle/``: pure Python integers and ``fractions.Fraction``,
with the fp32 and fp16 roundings written out from the IEEE-754 definition
(round to nearest, ties to even) instead of taken from numpy. Used to pin the
oracle on shapes small enough for per-element Python loops.

Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers
at Scale" (paper-graph-ui digest); [TM] transformer-math LLM.int8() tutorial
(aicassindra.com).
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple

Matrix = List[List[Fraction]]


def _round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _round_to_binary(q: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Nearest-even rounding of q to a binary format with ``mant_bits``
    significand bits (hidden bit included) and minimum normal exponent emin.
    Overflow is not modelled (callers stay far inside the range)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    step = Fraction(2) ** (e - (mant_bits - 1))
    n = _round_half_even(a / step)
    return sign * n * step


def fl32(q: Fraction) -> Fraction:
    return _round_to_binary(q, 24, -126)


def fl16(q: Fraction) -> Fraction:
    return _round_to_binary(q, 11, -14)


def half_away(q: Fraction) -> int:
    """Round to nearest integer, ties away from zero."""
    a = abs(q)
    n = (a + Fraction(1, 2)).numerator // (a + Fraction(1, 2)).denominator
    return n if q >= 0 else -n


def to_fractions(A) -> Matrix:
    return [[Fraction(float(v)) for v in row] for row in A]


def brute_force(X, W, alpha: float, bias=None) -> Tuple[List[int], List[Fraction], List[List[int]],
                                                         List[Fraction], List[List[int]], List[List[int]],
                                                         List[List[Fraction]]]:
    """Return (O, c_x, Xq, c_w, Wq [h][o], C_i32, C) for fp16-valued X [s][h], W [h][o]
    (and an optional fp16-valued bias [o], added to each row before rounding)."""
    Xf = to_fractions(X)
    Wf = to_fractions(W)
    s, h = len(Xf), len(Xf[0])
    o = len(Wf[0])
    a = Fraction(float(alpha)) if alpha != float("inf") else None
    # [DIGEST] Step 1: a column is an outlier if some |X_ij| >= alpha.
    O = [j for j in range(h) if a is not None and any(abs(Xf[i][j]) >= a for i in range(s))]
    Oset = set(O)
    # [DIGEST] Step 4: row scales over the non-outlier columns, then quantise.
    c_x: List[Fraction] = []
    Xq: List[List[int]] = []
    for i in range(s):
        regular = [abs(Xf[i][j]) for j in range(h) if j not in Oset]
        m = max(regular) if regular else Fraction(0)
        c = fl32(Fraction(127) / m) if m != 0 else Fraction(1)
        c_x.append(c)
        row = []
        for j in range(h):
            if j in Oset:
                row.append(0)
            else:
                row.append(max(-127, min(127, half_away(fl32(Xf[i][j] * c)))))
        Xq.append(row)
    # Column scales over all rows of W (load-time constants).
    c_w: List[Fraction] = []
    Wq = [[0] * o for _ in range(h)]
    for j in range(o):
        m = max(abs(Wf[i][j]) for i in range(h))
        c = fl32(Fraction(127) / m) if m != 0 else Fraction(1)
        c_w.append(c)
        for i in range(h):
            Wq[i][j] = max(-127, min(127, half_away(fl32(Wf[i][j] * c))))
    C_i32 = [[sum(Xq[i][k] * Wq[k][j] for k in range(h)) for j in range(o)] for i in range(s)]
    # [DIGEST] Steps 3-5: dequantise by 1/(c_x c_w), add the fp16 outlier product.
    C = []
    for i in range(s):
        row = []
        for j in range(o):
            v = Fraction(C_i32[i][j]) / (c_x[i] * c_w[j])
            v += sum((Xf[i][k] * Wf[k][j] for k in O), Fraction(0))
            if bias is not None:
                v += Fraction(float(bias[j]))
            row.append(fl16(v))
        C.append(row)
    return O, c_x, Xq, c_w, Wq, C_i32, C


def ulp16(v: Fraction) -> Fraction:
    """Spacing of fp16 numbers at |v| (2**-24 in the subnormal range)."""
    a = abs(v)
    if a < Fraction(2) ** -14:
        return Fraction(2) ** -24
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return Fraction(2) ** (e - 10)


def as_fractions_1d(v: Sequence[float]) -> List[Fraction]:
    return [Fraction(float(x)) for x in v]


def zeropoint_brute_force(X, W, alpha: float):
    """Zeropoint vector-wise with the decomposition, every step in exact
    rationals with IEEE rounding emulated (fl32 / fl16 above): returns
    (O, nd_x, zp_x, Xq, nd_w, zp_w, Wq [h][o], C' [s][o], C [s][o]).
    nd = fl32(254 / fl32(max - min)) (1 if max == min); zp = round(fl32(nd
    min)) + 127; q = clamp(round(fl32(nd x)) - zp, -127, 127); C' is the sum
    over the non-outlier columns of the shifted codes' products and
    C = fl16(C' / (nd_x nd_w) + sum over O of X W)."""
    Xf = to_fractions(X)
    Wf = to_fractions(W)
    s, h = len(Xf), len(Xf[0])
    o = len(Wf[0])
    a = Fraction(float(alpha)) if alpha != float("inf") else None
    O = [j for j in range(h) if a is not None and any(abs(Xf[i][j]) >= a for i in range(s))]
    reg = [j for j in range(h) if j not in set(O)]

    def params(vals):
        lo, hi = (min(vals), max(vals)) if vals else (Fraction(0), Fraction(0))
        span = fl32(hi - lo)
        nd = fl32(Fraction(254) / span) if span != 0 else Fraction(1)
        return nd, half_away(fl32(nd * lo)) + 127

    def code(x, nd, zp):
        return max(-127, min(127, half_away(fl32(nd * x)) - zp))

    nd_x, zp_x, Xq = [], [], []
    for i in range(s):
        nd, zp = params([Xf[i][j] for j in reg])
        nd_x.append(nd)
        zp_x.append(zp)
        Xq.append([code(Xf[i][j], nd, zp) if j in reg else 0 for j in range(h)])
    nd_w, zp_w = [], []
    Wq = [[0] * o for _ in range(h)]
    for j in range(o):
        nd, zp = params([Wf[k][j] for k in range(h)])
        nd_w.append(nd)
        zp_w.append(zp)
        for k in range(h):
            Wq[k][j] = code(Wf[k][j], nd, zp)
    Cp = [[sum((Xq[i][k] + zp_x[i]) * (Wq[k][j] + zp_w[j]) for k in reg) for j in range(o)] for i in range(s)]
    C = [[fl16(Fraction(Cp[i][j]) / (nd_x[i] * nd_w[j]) + sum((Xf[i][k] * Wf[k][j] for k in O), Fraction(0)))
          for j in range(o)] for i in range(s)]
    return O, nd_x, zp_x, Xq, nd_w, zp_w, Wq, Cp, C
