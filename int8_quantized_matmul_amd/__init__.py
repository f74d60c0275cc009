"""LLM.int8() mixed-precision decomposed int8 matmul for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libi8mm.so (include/i8mm.h). Each
function checks tensor placement, dtype and shape, allocates outputs with
torch on the tensors' device, and passes raw device pointers plus torch's
current HIP stream to the library. Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback: without the
built library the first call raises ImportError.

Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers
at Scale" (paper-graph-ui digest), "The Full LLM.int8() Algorithm".
"""

from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple

import torch

from . import _native

__all__ = [
    "quantize_colwise_weights",
    "detect_outlier_cols",
    "quantize_rowwise",
    "int8_mixed_matmul",
    "outlier_matmul",
    "int8_gemm_i32",
    "forward",
    "forward_tensorwise",
    "forward_zeropoint",
    "forward_noalloc",
    "forward_decode",
    "forward_inline_quant",
    "INLINE_QUANT_MIN_ROWS",
    "NOALLOC_SCRATCH_BYTES",
    "pack_fp16_weights",
    "fp16_gemm",
    "quantize_tensorwise",
    "quantize_weights_tensorwise",
    "quantize_rowwise_zeropoint",
    "quantize_colwise_weights_zeropoint",
    "zeropoint_matmul",
    "SCHEMES",
    "quantize_weights",
    "variant_forward",
    "forward_workspace",
    "forward_workspace_views",
    "x_o_stride",
    "weight_panels_shape",
    "panels_to_rows",
    "version",
    "library_path",
    "I8MMError",
]


class _LazyLib:
    """Loads libi8mm.so on first use, so that the build module can be imported
    before the library exists. Any call without the library raises ImportError."""

    def __getattr__(self, name):
        return getattr(_native.load(), name)


_lib = _LazyLib()

# Bytes of the forward workspace's leading accumulator (I8MM_FORWARD_ACC_BYTES).
ACC_BYTES = _native.header_define("I8MM_FORWARD_ACC_BYTES")
# Bytes of the static device scratch behind forward_noalloc (I8MM_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = _native.header_define("I8MM_NOALLOC_SCRATCH_BYTES")
# Fewest rows forward_inline_quant takes (I8MM_INLINE_QUANT_MIN_ROWS).
INLINE_QUANT_MIN_ROWS = _native.header_define("I8MM_INLINE_QUANT_MIN_ROWS")


class I8MMError(RuntimeError):
    """A libi8mm entry point returned an error status."""


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _lib.i8mm_status_string(status).decode()
        raise I8MMError(f"{what}: {msg} (status {status})")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def x_o_stride(h: int) -> int:
    """Row stride (elements) of the gathered outlier columns X_O: room for |O| = h."""
    return (h + 31) // 32 * 32


def weight_panels_shape(h: int, o: int) -> Tuple[int, int, int]:
    """Shape of the quantised weights in the library's panel layout: the code
    W_i8[k, j] sits at Wq[k // 64, j, k % 64] (h / 64 panels of 64 reduction
    rows, each column's 64 codes contiguous)."""
    if h % 64 != 0:
        raise ValueError(f"h must be a multiple of 64 (got {h})")
    return (h // 64, o, 64)


def panels_to_rows(Wq: torch.Tensor) -> torch.Tensor:
    """The codes of a panel-layout Wq as W_i8 transposed, [o, h] (a copy, for
    inspection and tests; the products read the panel layout directly)."""
    p, o, _ = Wq.shape
    return Wq.permute(1, 0, 2).reshape(o, p * 64)


def version() -> str:
    return _lib.i8mm_version().decode()


def library_path() -> str:
    return _native.loaded_path()


def quantize_colwise_weights(W: torch.Tensor, Wq: Optional[torch.Tensor] = None,
                             c_w: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Load-time conversion: W fp16 [h, o] -> (Wq int8 [h/64, o, 64] panel
    layout, c_w fp32 [o])."""
    h, o = W.shape
    shape = weight_panels_shape(h, o)
    if Wq is None:
        Wq = torch.empty(shape, dtype=torch.int8, device=W.device)
    if c_w is None:
        c_w = torch.empty((o,), dtype=torch.float32, device=W.device)
    st = _lib.i8mm_quantize_colwise_weights(
        _dev(W, "W", torch.float16), h, o, _dev(Wq, "Wq", torch.int8, shape),
        _dev(c_w, "c_w", torch.float32, (o,)), _stream(W))
    _check(st, "quantize_colwise_weights")
    return Wq, c_w


def detect_outlier_cols(X: torch.Tensor, alpha: float = 6.0, mask: Optional[torch.Tensor] = None,
                        idx: Optional[torch.Tensor] = None, n_out: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """O = {j : max_i |X_ij| >= alpha} as (mask int32 view of uint32 [ceil(h/32)],
    idx int32 [h] (first |O| valid, ascending), n_out int32 [1]) on the device."""
    s, h = X.shape
    nw = (h + 31) // 32
    dev = X.device
    if mask is None:
        mask = torch.empty((nw,), dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty((h,), dtype=torch.int32, device=dev)
    if n_out is None:
        n_out = torch.empty((1,), dtype=torch.int32, device=dev)
    st = _lib.i8mm_detect_outlier_cols(
        _dev(X, "X", torch.float16), s, h, float(alpha), _dev(mask, "mask", torch.int32, (nw,)),
        _dev(idx, "idx", torch.int32, (h,)), _dev(n_out, "n_out", torch.int32, (1,)), _stream(X))
    _check(st, "detect_outlier_cols")
    return mask, idx, n_out


def quantize_rowwise(X: torch.Tensor, mask: torch.Tensor, idx: torch.Tensor, n_out: torch.Tensor,
                     Xq: Optional[torch.Tensor] = None, c_x: Optional[torch.Tensor] = None,
                     X_O: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Row-wise absmax int8 over the non-outlier columns: (Xq int8 [s, h] with
    O columns 0, c_x fp32 [s], X_O fp16 [s, x_o_stride(h)] gathered outliers)."""
    s, h = X.shape
    dev = X.device
    ldo = x_o_stride(h) if X_O is None else X_O.shape[1]
    if Xq is None:
        Xq = torch.empty((s, h), dtype=torch.int8, device=dev)
    if c_x is None:
        c_x = torch.empty((s,), dtype=torch.float32, device=dev)
    if X_O is None:
        X_O = torch.empty((s, ldo), dtype=torch.float16, device=dev)
    st = _lib.i8mm_quantize_rowwise(
        _dev(X, "X", torch.float16), s, h, _dev(mask, "mask", torch.int32),
        _dev(idx, "idx", torch.int32), _dev(n_out, "n_out", torch.int32, (1,)),
        _dev(Xq, "Xq", torch.int8, (s, h)), _dev(c_x, "c_x", torch.float32, (s,)),
        _dev(X_O, "X_O", torch.float16, (s, ldo)), ldo, _stream(X))
    _check(st, "quantize_rowwise")
    return Xq, c_x, X_O


def _weights_ptr(W: Optional[torch.Tensor], h: int, o: int) -> Optional[int]:
    """Pointer of the resident fp16 W, or None (outlier rows rebuilt from Wq / c_w)."""
    return None if W is None else _dev(W, "W", torch.float16, (h, o))


def _bias_ptr(bias: Optional[torch.Tensor], o: int) -> Optional[int]:
    """Pointer of the fp16 layer bias [o], or None (no bias)."""
    return None if bias is None else _dev(bias, "bias", torch.float16, (o,))


def int8_mixed_matmul(Xq: torch.Tensor, c_x: torch.Tensor, X_O: torch.Tensor, idx: torch.Tensor,
                      n_out: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
                      C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C fp16 [s, o] = fp16(C_i32 / (c_x ⊗ c_w) + X_O W[idx, :] [+ bias]). With W
    None no fp16 copy of the weights is needed: W[idx, :] is rebuilt as
    fp16(W_i8 * fl32(1 / c_w)). bias: fp16 [o] or None."""
    s, h = Xq.shape
    o = Wq.shape[1]
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=Xq.device)
    st = _lib.i8mm_int8_mixed_matmul(
        _dev(Xq, "Xq", torch.int8), _dev(c_x, "c_x", torch.float32, (s,)),
        _dev(X_O, "X_O", torch.float16), X_O.shape[1], _dev(idx, "idx", torch.int32),
        _dev(n_out, "n_out", torch.int32, (1,)), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        s, h, o, _dev(C, "C", torch.float16, (s, o)), _stream(Xq))
    _check(st, "int8_mixed_matmul")
    return C


def outlier_matmul(X_O: torch.Tensor, idx: torch.Tensor, n_out: torch.Tensor, W: torch.Tensor,
                   C_O: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C_O fp32 [s, o] = X_O W[idx, :] (the fp16 outlier product alone)."""
    s, ldo = X_O.shape
    h, o = W.shape
    if C_O is None:
        C_O = torch.empty((s, o), dtype=torch.float32, device=X_O.device)
    st = _lib.i8mm_outlier_matmul(
        _dev(X_O, "X_O", torch.float16), ldo, _dev(idx, "idx", torch.int32),
        _dev(n_out, "n_out", torch.int32, (1,)), _dev(W, "W", torch.float16), s, h, o,
        _dev(C_O, "C_O", torch.float32, (s, o)), _stream(X_O))
    _check(st, "outlier_matmul")
    return C_O


def int8_gemm_i32(Xq: torch.Tensor, Wq: torch.Tensor, C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C_i32 int32 [s, o] = Xq W_i8 exactly (same main loop as the mixed product)."""
    s, h = Xq.shape
    o = Wq.shape[1]
    if C is None:
        C = torch.empty((s, o), dtype=torch.int32, device=Xq.device)
    st = _lib.i8mm_int8_gemm_i32(
        _dev(Xq, "Xq", torch.int8), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)), s, h, o,
        _dev(C, "C", torch.int32, (s, o)), _stream(Xq))
    _check(st, "int8_gemm_i32")
    return C


def pack_fp16_weights(W: torch.Tensor, Wp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Load-time packing for the dense fp16 baseline: W fp16 [h, o] -> Wp fp16
    [h/32, o, 32] (W[k, j] at Wp[k // 32, j, k % 32])."""
    h, o = W.shape
    if h % 32 != 0:
        raise ValueError(f"h must be a multiple of 64 (got {h})")
    shape = (h // 32, o, 32)
    if Wp is None:
        Wp = torch.empty(shape, dtype=torch.float16, device=W.device)
    st = _lib.i8mm_pack_fp16_weights(_dev(W, "W", torch.float16), h, o, _dev(Wp, "Wp", torch.float16, shape),
                                     _stream(W))
    _check(st, "pack_fp16_weights")
    return Wp


def fp16_gemm(X: torch.Tensor, Wp: torch.Tensor, C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense fp16 baseline C fp16 [s, o] = fp16(X W) (fp32 accumulation) from packed Wp."""
    s, h = X.shape
    o = Wp.shape[1]
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    st = _lib.i8mm_fp16_gemm(_dev(X, "X", torch.float16), _dev(Wp, "Wp", torch.float16, (h // 32, o, 32)),
                             s, h, o, _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "fp16_gemm")
    return C


# ---------------------------------------------------------------- quantiser variants (Table 1)

def quantize_weights_tensorwise(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tensor-wise absmax for W: (Wq int8 panels, c_w fp32 [o] all equal to the
    one constant 127 / max |W|)."""
    h, o = W.shape
    Wq = torch.empty(weight_panels_shape(h, o), dtype=torch.int8, device=W.device)
    c_w = torch.empty((o,), dtype=torch.float32, device=W.device)
    st = _lib.i8mm_quantize_weights_tensorwise(_dev(W, "W", torch.float16), h, o, _dev(Wq, "Wq", torch.int8),
                                               _dev(c_w, "c_w", torch.float32), _stream(W))
    _check(st, "quantize_weights_tensorwise")
    return Wq, c_w


def quantize_tensorwise(X: torch.Tensor, mask: torch.Tensor, idx: torch.Tensor, n_out: torch.Tensor
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Tensor-wise absmax for X over the non-outlier columns: (Xq, c_x [s] all
    equal, X_O), laid out as by quantize_rowwise."""
    s, h = X.shape
    dev = X.device
    ldo = x_o_stride(h)
    Xq = torch.empty((s, h), dtype=torch.int8, device=dev)
    c_x = torch.empty((s,), dtype=torch.float32, device=dev)
    X_O = torch.empty((s, ldo), dtype=torch.float16, device=dev)
    st = _lib.i8mm_quantize_tensorwise(
        _dev(X, "X", torch.float16), s, h, _dev(mask, "mask", torch.int32), _dev(idx, "idx", torch.int32),
        _dev(n_out, "n_out", torch.int32, (1,)), _dev(Xq, "Xq", torch.int8), _dev(c_x, "c_x", torch.float32),
        _dev(X_O, "X_O", torch.float16), ldo, _stream(X))
    _check(st, "quantize_tensorwise")
    return Xq, c_x, X_O


def quantize_colwise_weights_zeropoint(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                                                 torch.Tensor]:
    """Zeropoint quantisation of the columns of W (load time): (Wq int8 panels,
    nd_w fp32 [o], zp_w int32 [o], colsum_w int32 [o])."""
    h, o = W.shape
    dev = W.device
    Wq = torch.empty(weight_panels_shape(h, o), dtype=torch.int8, device=dev)
    nd_w = torch.empty((o,), dtype=torch.float32, device=dev)
    zp_w = torch.empty((o,), dtype=torch.int32, device=dev)
    cs_w = torch.empty((o,), dtype=torch.int32, device=dev)
    st = _lib.i8mm_quantize_colwise_weights_zeropoint(
        _dev(W, "W", torch.float16), h, o, _dev(Wq, "Wq", torch.int8), _dev(nd_w, "nd_w", torch.float32),
        _dev(zp_w, "zp_w", torch.int32), _dev(cs_w, "colsum_w", torch.int32), _stream(W))
    _check(st, "quantize_colwise_weights_zeropoint")
    return Wq, nd_w, zp_w, cs_w


def quantize_rowwise_zeropoint(X: torch.Tensor, mask: torch.Tensor, idx: torch.Tensor, n_out: torch.Tensor
                               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """Zeropoint quantisation of the rows of X over the non-outlier columns:
    (Xq int8 [s, h], nd_x fp32 [s], zp_x int32 [s], rowsum_x int32 [s], X_O)."""
    s, h = X.shape
    dev = X.device
    ldo = x_o_stride(h)
    Xq = torch.empty((s, h), dtype=torch.int8, device=dev)
    nd_x = torch.empty((s,), dtype=torch.float32, device=dev)
    zp_x = torch.empty((s,), dtype=torch.int32, device=dev)
    rs_x = torch.empty((s,), dtype=torch.int32, device=dev)
    X_O = torch.empty((s, ldo), dtype=torch.float16, device=dev)
    st = _lib.i8mm_quantize_rowwise_zeropoint(
        _dev(X, "X", torch.float16), s, h, _dev(mask, "mask", torch.int32), _dev(idx, "idx", torch.int32),
        _dev(n_out, "n_out", torch.int32, (1,)), _dev(Xq, "Xq", torch.int8), _dev(nd_x, "nd_x", torch.float32),
        _dev(zp_x, "zp_x", torch.int32), _dev(rs_x, "rowsum_x", torch.int32), _dev(X_O, "X_O", torch.float16), ldo,
        _stream(X))
    _check(st, "quantize_rowwise_zeropoint")
    return Xq, nd_x, zp_x, rs_x, X_O


def zeropoint_matmul(Xq: torch.Tensor, nd_x: torch.Tensor, zp_x: torch.Tensor, rowsum_x: torch.Tensor,
                     X_O: torch.Tensor, idx: torch.Tensor, n_out: torch.Tensor, Wq: torch.Tensor,
                     nd_w: torch.Tensor, zp_w: torch.Tensor, colsum_w: torch.Tensor, W: torch.Tensor,
                     C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C fp16 [s, o] = fp16(C' / (nd_x ⊗ nd_w) + X_O W[idx, :] [+ bias]), C' the
    product of the zero-point-shifted codes over the non-outlier columns."""
    s, h = Xq.shape
    o = Wq.shape[1]
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=Xq.device)
    st = _lib.i8mm_zeropoint_matmul(
        _dev(Xq, "Xq", torch.int8), _dev(nd_x, "nd_x", torch.float32, (s,)), _dev(zp_x, "zp_x", torch.int32, (s,)),
        _dev(rowsum_x, "rowsum_x", torch.int32, (s,)), _dev(X_O, "X_O", torch.float16), X_O.shape[1],
        _dev(idx, "idx", torch.int32), _dev(n_out, "n_out", torch.int32, (1,)),
        _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)), _dev(nd_w, "nd_w", torch.float32, (o,)),
        _dev(zp_w, "zp_w", torch.int32, (o,)), _dev(colsum_w, "colsum_w", torch.int32, (o,)),
        _dev(W, "W", torch.float16, (h, o)), _bias_ptr(bias, o), s, h, o, _dev(C, "C", torch.float16, (s, o)),
        _stream(Xq))
    _check(st, "zeropoint_matmul")
    return C


SCHEMES = ("tensor", "row", "vector", "zeropoint")


def quantize_weights(W: torch.Tensor, scheme: str) -> Tuple[torch.Tensor, ...]:
    """Load-time weights for one quantiser scheme: (Wq, c_w) for "tensor" and
    "row" (one constant) and "vector" (per column); (Wq, nd_w, zp_w, colsum_w)
    for "zeropoint"."""
    if scheme in ("tensor", "row"):
        return quantize_weights_tensorwise(W)
    if scheme == "vector":
        return quantize_colwise_weights(W)
    if scheme == "zeropoint":
        return quantize_colwise_weights_zeropoint(W)
    raise ValueError(f"unknown scheme {scheme!r}; one of {SCHEMES}")


def variant_forward(X: torch.Tensor, qw: Tuple[torch.Tensor, ...], W: torch.Tensor, scheme: str,
                    alpha: float = 6.0, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One forward of a quantiser scheme (Table 1) as a sequence of C-ABI
    calls: detection at alpha (inf: no decomposition), the scheme's row
    quantiser, then its product. qw comes from quantize_weights(W, scheme)."""
    mask, idx, n_out = detect_outlier_cols(X, alpha)
    if scheme == "zeropoint":
        Xq, nd_x, zp_x, rs_x, X_O = quantize_rowwise_zeropoint(X, mask, idx, n_out)
        Wq, nd_w, zp_w, cs_w = qw
        return zeropoint_matmul(Xq, nd_x, zp_x, rs_x, X_O, idx, n_out, Wq, nd_w, zp_w, cs_w, W, bias=bias)
    if scheme == "tensor":
        Xq, c_x, X_O = quantize_tensorwise(X, mask, idx, n_out)
    elif scheme in ("row", "vector"):
        Xq, c_x, X_O = quantize_rowwise(X, mask, idx, n_out)
    else:
        raise ValueError(f"unknown scheme {scheme!r}; one of {SCHEMES}")
    Wq, c_w = qw
    return int8_mixed_matmul(Xq, c_x, X_O, idx, n_out, Wq, c_w, W, bias=bias)


def forward_workspace(s: int, h: int, device, zeropoint: bool = False) -> torch.Tensor:
    """A zero-filled device workspace (uint8) for forward() and
    forward_tensorwise() (zeropoint=True: sized for forward_zeropoint(),
    which also serves the others). Its leading accumulator must start at
    zero; every one-call forward leaves it zero again."""
    n = (_lib.i8mm_forward_zeropoint_workspace_bytes if zeropoint else _lib.i8mm_forward_workspace_bytes)(s, h)
    if n == 0:
        raise I8MMError(f"invalid shape for the forward workspace: s={s}, h={h}")
    return torch.zeros((n,), dtype=torch.uint8, device=device)


def forward_workspace_views(workspace: torch.Tensor, s: int, h: int) -> Dict[str, torch.Tensor]:
    """Typed views of the intermediates that forward() leaves in its workspace."""
    offs = (ctypes.c_size_t * 7)()
    ldo = ctypes.c_int64()
    _check(_lib.i8mm_forward_workspace_layout(s, h, offs, ctypes.byref(ldo)), "forward_workspace_layout")
    nw = (h + 31) // 32
    l = ldo.value

    def view(i, nbytes, dtype, shape):
        return workspace[offs[i]:offs[i] + nbytes].view(dtype).view(shape)

    acc_words = ACC_BYTES // 4
    return {
        "acc": view(0, ACC_BYTES, torch.int32, (acc_words,)),
        "mask": view(1, 4 * nw, torch.int32, (nw,)),
        "idx": view(2, 4 * h, torch.int32, (h,)),
        "n_out": view(3, 4, torch.int32, (1,)),
        "Xq": view(4, s * h, torch.int8, (s, h)),
        "c_x": view(5, 4 * s, torch.float32, (s,)),
        "X_O": view(6, 2 * s * l, torch.float16, (s, l)),
    }


def forward(X: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
            alpha: float = 6.0, workspace: Optional[torch.Tensor] = None,
            C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole per-forward path: detect -> quantise rows -> decomposed product.
    W is the resident fp16 weight matrix, or None (outlier rows rebuilt from
    Wq / c_w); bias is the fp16 layer bias [o], or None."""
    s, h = X.shape
    o = Wq.shape[1]
    if workspace is None:
        workspace = forward_workspace(s, h, X.device)
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    need = _lib.i8mm_forward_workspace_bytes(s, h)
    if workspace.numel() < need or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    st = _lib.i8mm_forward(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        _dev(workspace, "workspace", torch.uint8), _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward")
    return C


def forward_tensorwise(X: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
                       alpha: float = 6.0, workspace: Optional[torch.Tensor] = None,
                       C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() with tensor-wise absmax for X (one constant over the columns
    not in O): Table 1's tensor-wise scheme with weights from
    quantize_weights_tensorwise (or quantize_weights(W, "tensor"))."""
    s, h = X.shape
    o = Wq.shape[1]
    if workspace is None:
        workspace = forward_workspace(s, h, X.device)
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    need = _lib.i8mm_forward_workspace_bytes(s, h)
    if workspace.numel() < need or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    st = _lib.i8mm_forward_tensorwise(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        _dev(workspace, "workspace", torch.uint8), _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward_tensorwise")
    return C


def forward_zeropoint(X: torch.Tensor, qw: Tuple[torch.Tensor, ...], W: torch.Tensor, alpha: float = 6.0,
                      workspace: Optional[torch.Tensor] = None, C: Optional[torch.Tensor] = None,
                      bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The one-call forward of the zeropoint vector-wise scheme: qw = (Wq,
    nd_w, zp_w, colsum_w) from quantize_weights(W, "zeropoint"); W (fp16) is
    required for the outlier rows. The workspace must come from
    forward_workspace(s, h, device, zeropoint=True) or be as large."""
    s, h = X.shape
    Wq, nd_w, zp_w, cs_w = qw
    o = Wq.shape[1]
    if workspace is None:
        workspace = forward_workspace(s, h, X.device, zeropoint=True)
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    need = _lib.i8mm_forward_zeropoint_workspace_bytes(s, h)
    if workspace.numel() < need or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    st = _lib.i8mm_forward_zeropoint(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(nd_w, "nd_w", torch.float32, (o,)), _dev(zp_w, "zp_w", torch.int32, (o,)),
        _dev(cs_w, "colsum_w", torch.int32, (o,)), _dev(W, "W", torch.float16, (h, o)), _bias_ptr(bias, o),
        _dev(workspace, "workspace", torch.uint8), _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward_zeropoint")
    return C


def forward_decode(X: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
                   alpha: float = 6.0, workspace: Optional[torch.Tensor] = None,
                   C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() in one kernel launch for s <= 16 rows (i8mm_forward_decode);
    the workspace receives the same intermediates as forward()'s."""
    s, h = X.shape
    o = Wq.shape[1]
    if workspace is None:
        workspace = forward_workspace(s, h, X.device)
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    need = _lib.i8mm_forward_workspace_bytes(s, h)
    if workspace.numel() < need or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    st = _lib.i8mm_forward_decode(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        _dev(workspace, "workspace", torch.uint8), _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward_decode")
    return C


def forward_inline_quant(X: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
                         alpha: float = 6.0, workspace: Optional[torch.Tensor] = None,
                         C: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() with the int8 codes of X made inside the product kernel
    and never stored (i8mm_forward_inline_quant; s >= INLINE_QUANT_MIN_ROWS).
    The workspace receives the outlier set, c_x and X_O; its Xq region is
    not written."""
    s, h = X.shape
    o = Wq.shape[1]
    if workspace is None:
        workspace = forward_workspace(s, h, X.device)
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    need = _lib.i8mm_forward_workspace_bytes(s, h)
    if workspace.numel() < need or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    st = _lib.i8mm_forward_inline_quant(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        _dev(workspace, "workspace", torch.uint8), _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward_inline_quant")
    return C


def forward_noalloc(X: torch.Tensor, Wq: torch.Tensor, c_w: torch.Tensor, W: Optional[torch.Tensor],
                    alpha: float = 6.0, C: torch.Tensor = None, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """forward() over the library's static device scratch instead of a
    workspace: the call allocates nothing on the device when C is given
    (for graph capture and loops that must not allocate). Raises I8MMError
    (status -5) when the shape needs more than NOALLOC_SCRATCH_BYTES of
    workspace. Calls on one GPU share the scratch and must not overlap."""
    s, h = X.shape
    o = Wq.shape[1]
    if C is None:
        C = torch.empty((s, o), dtype=torch.float16, device=X.device)
    st = _lib.i8mm_forward_noalloc(
        _dev(X, "X", torch.float16), s, h, o, float(alpha), _dev(Wq, "Wq", torch.int8, weight_panels_shape(h, o)),
        _dev(c_w, "c_w", torch.float32, (o,)), _weights_ptr(W, h, o), _bias_ptr(bias, o),
        _dev(C, "C", torch.float16, (s, o)), _stream(X))
    _check(st, "forward_noalloc")
    return C


def calib_mfma_i8(codes: torch.Tensor, iters: int, out: torch.Tensor) -> int:
    """Measurement calibration (not the method): enqueues a stream of int8
    MFMAs on register-resident operands, len(out) / 256 blocks of four
    wavefronts, 32 * iters MFMAs per wavefront. codes: int8, 65536 per block;
    out: int32, 256 per block. Returns the integer operations performed."""
    blocks = out.numel() // 256
    if blocks < 1 or out.numel() != blocks * 256:
        raise ValueError("out must hold a positive multiple of 256 int32")
    st = _lib.i8mm_calib_mfma_i8(_dev(codes, "codes", torch.int8, (blocks * 65536,)), blocks, iters,
                                 _dev(out, "out", torch.int32, (blocks * 256,)), _stream(codes))
    _check(st, "calib_mfma_i8")
    return blocks * 4 * 32 * iters * 65536
