"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before touching any device (runs without a GPU)."""

import ctypes
import os

import pytest

from int8_quantized_matmul_amd import _native


def _lib():
    if not os.path.exists(_native.LIB_PATH):
        from int8_quantized_matmul_amd.build import build
        build()
    return _native.load()


def test_exports_every_declared_symbol():
    lib = _lib()
    names = _native.header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(_native._SIGNATURES) == set(names)


def test_version_and_status_strings():
    lib = _lib()
    assert b"gfx950" in lib.i8mm_version()
    assert lib.i8mm_status_string(0) == b"ok"
    assert lib.i8mm_status_string(-1) == b"invalid argument"
    assert lib.i8mm_status_string(-2) == b"no gfx950 device"
    assert lib.i8mm_status_string(-3) == b"kernel launch failed"
    assert b"workspace accumulator" in lib.i8mm_status_string(-4)
    assert lib.i8mm_status_string(-99) == b"unknown status"


def test_forward_error_contract_is_declared():
    """The one-call forwards' error path as the header states it: a failed
    launch after the detection returns I8MM_ELAUNCH with the accumulator
    cleared by one more launch, or I8MM_EWORKSPACE if that launch fails too;
    the test hook that forces the failure from the host is exported."""
    with open(_native.HEADER) as f:
        text = f.read()
    assert "I8MM_EWORKSPACE = -4" in text
    assert "clears the accumulator and the call returns I8MM_ELAUNCH" in text
    lib = _lib()
    lib.i8mm_test_fail_product_launches(0)   # host-only: sets nothing on a device
    # with no device the check comes first and leaves the hook untouched
    import torch
    if torch.cuda.device_count() == 0:
        lib.i8mm_test_fail_product_launches(1)
        ws = ctypes.c_void_p(1 << 20)
        assert lib.i8mm_forward(P, 4, 64, 64, 6.0, P, P, P, None, ws, P, None) == -2
        lib.i8mm_test_fail_product_launches(0)


P = ctypes.c_void_p(1 << 20)          # a 16-byte aligned non-null stand-in (never dereferenced)
MIS = ctypes.c_void_p((1 << 20) + 4)  # misaligned


@pytest.mark.parametrize("args", [
    (None, 64, 64, P, P, None),       # null W
    (P, 63, 64, P, P, None),          # h not a multiple of 64
    (P, 64, 96, P, P, None),          # o not a multiple of 64
    (P, 133184, 64, P, P, None),      # h above the int32 bound
    (MIS, 64, 64, P, P, None),        # misaligned
])
def test_quantize_colwise_weights_rejects(args):
    assert _lib().i8mm_quantize_colwise_weights(*args) == -1


@pytest.mark.parametrize("s,h,alpha", [(0, 64, 6.0), (4, 0, 6.0), (4, 100, 6.0), (4, 64, float("nan")),
                                       (4, 64, -1.0)])
def test_detect_rejects(s, h, alpha):
    assert _lib().i8mm_detect_outlier_cols(P, s, h, alpha, P, P, P, None) == -1


def test_quantize_rowwise_rejects_small_ldo():
    lib = _lib()
    assert lib.i8mm_quantize_rowwise(P, 4, 128, P, P, P, P, P, P, 96, None) == -1   # ldo < h
    assert lib.i8mm_quantize_rowwise(P, 4, 128, P, P, P, P, P, P, 132, None) == -1  # ldo % 8
    assert lib.i8mm_quantize_rowwise(P, 4, 128, P, P, None, P, P, P, 128, None) == -1


def test_mixed_matmul_and_gemm_reject():
    lib = _lib()
    assert lib.i8mm_int8_mixed_matmul(P, P, P, 64, P, P, P, P, P, None, 4, 64, 64, None, None) == -1
    assert lib.i8mm_int8_mixed_matmul(P, P, P, 32, P, P, P, P, P, None, 4, 64, 64, P, None) == -1
    # a misaligned bias
    assert lib.i8mm_int8_mixed_matmul(P, P, P, 64, P, P, P, P, P, MIS, 4, 64, 64, P, None) == -1
    assert lib.i8mm_int8_gemm_i32(P, P, 4, 64, 65, P, None) == -1
    # W larger than 32-bit byte offsets can address (h * o >= 2^31)
    assert lib.i8mm_int8_mixed_matmul(P, P, P, 65536, P, P, P, P, P, None, 4, 65536, 32768, P, None) == -1
    assert lib.i8mm_int8_gemm_i32(P, P, 4, 65536, 32768, P, None) == -1
    assert lib.i8mm_outlier_matmul(P, 64, P, P, P, 4, 64, 64, MIS, None) == -1


def test_single_launch_decode_rejects():
    lib = _lib()
    ws = ctypes.c_void_p(1 << 20)
    # more rows than the single launch takes; null workspace; misaligned bias
    assert lib.i8mm_forward_decode(P, 17, 64, 64, 6.0, P, P, P, None, ws, P, None) == -1
    assert lib.i8mm_forward_decode(P, 8, 64, 64, 6.0, P, P, P, None, None, P, None) == -1
    assert lib.i8mm_forward_decode(P, 8, 64, 64, 6.0, P, P, P, MIS, ws, P, None) == -1


def test_forward_rejects_unaligned_workspace():
    lib = _lib()
    ws = ctypes.c_void_p((1 << 20) + 16)
    assert lib.i8mm_forward(P, 4, 64, 64, 6.0, P, P, P, None, ws, P, None) == -1
    # a misaligned bias
    assert lib.i8mm_forward(P, 4, 64, 64, 6.0, P, P, P, MIS, ctypes.c_void_p(1 << 20), P, None) == -1


def test_variant_forwards_reject():
    lib = _lib()
    ws = ctypes.c_void_p(1 << 20)
    # unaligned workspace, misaligned bias, null weights
    assert lib.i8mm_forward_tensorwise(P, 4, 64, 64, 6.0, P, P, P, None, ctypes.c_void_p((1 << 20) + 16), P,
                                       None) == -1
    assert lib.i8mm_forward_tensorwise(P, 4, 64, 64, 6.0, P, P, P, MIS, ws, P, None) == -1
    assert lib.i8mm_forward_tensorwise(P, 4, 64, 64, 6.0, None, P, P, None, ws, P, None) == -1
    assert lib.i8mm_forward_tensorwise(P, 4, 64, 64, float("nan"), P, P, P, None, ws, P, None) == -1
    # zeropoint: W is required; bad shape; NaN alpha
    assert lib.i8mm_forward_zeropoint(P, 4, 64, 64, 6.0, P, P, P, P, None, None, ws, P, None) == -1
    assert lib.i8mm_forward_zeropoint(P, 4, 96, 64, 6.0, P, P, P, P, P, None, ws, P, None) == -1
    assert lib.i8mm_forward_zeropoint(P, 4, 64, 64, -1.0, P, P, P, P, P, None, ws, P, None) == -1
    for s, h in [(1, 64), (2048, 4096), (3, 133120)]:
        extra = 2 * ((4 * s + 255) // 256 * 256)
        assert lib.i8mm_forward_zeropoint_workspace_bytes(s, h) == lib.i8mm_forward_workspace_bytes(s, h) + extra
    assert lib.i8mm_forward_zeropoint_workspace_bytes(0, 64) == 0


def test_forward_workspace_layout():
    lib = _lib()
    for s, h in [(1, 64), (16, 256), (2048, 4096), (4096, 12288), (3, 133120)]:
        total = lib.i8mm_forward_workspace_bytes(s, h)
        offs = (ctypes.c_size_t * 7)()
        ldo = ctypes.c_int64()
        assert lib.i8mm_forward_workspace_layout(s, h, offs, ctypes.byref(ldo)) == 0
        assert ldo.value == (h + 31) // 32 * 32
        assert offs[0] == 0   # the accumulator sits first, whatever the shape
        sizes = [16640, 4 * ((h + 31) // 32), 4 * h, 4, s * h, 4 * s, 2 * s * ldo.value]
        assert 16640 >= 4 * (133120 // 32)
        for i in range(7):
            assert offs[i] % 256 == 0
            end = offs[i] + sizes[i]
            assert end <= (offs[i + 1] if i < 6 else total)
    assert lib.i8mm_forward_workspace_bytes(0, 64) == 0
    assert lib.i8mm_forward_workspace_bytes(4, 96) == 0


def test_valid_call_without_gpu_reports_no_device():
    """With valid arguments the call reaches the device check; on a machine
    with no GPU that is I8MM_EDEVICE (nothing is enqueued)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert _lib().i8mm_int8_gemm_i32(P, P, 1, 64, 64, P, None) == -2


def test_variant_entry_points_reject():
    """The quantiser variants validate like the main entry points."""
    lib = _lib()
    assert lib.i8mm_quantize_tensorwise(P, 4, 128, P, P, P, P, P, P, 96, None) == -1        # ldo < h
    assert lib.i8mm_quantize_tensorwise(P, 4, 100, P, P, P, P, P, P, 128, None) == -1       # h % 64
    assert lib.i8mm_quantize_weights_tensorwise(P, 64, 65, P, P, None) == -1
    assert lib.i8mm_quantize_weights_tensorwise(P, 64, 64, MIS, P, None) == -1
    assert lib.i8mm_quantize_rowwise_zeropoint(P, 4, 128, P, P, P, P, P, None, P, P, 128, None) == -1
    assert lib.i8mm_quantize_rowwise_zeropoint(P, 4, 128, P, P, P, P, P, P, P, P, 132, None) == -1
    assert lib.i8mm_quantize_colwise_weights_zeropoint(P, 64, 64, P, P, P, None, None) == -1
    assert lib.i8mm_quantize_colwise_weights_zeropoint(P, 96, 64, P, P, P, P, None) == -1
    # W is required by the zeropoint product; bias must be aligned
    args = [P, P, P, P, P, 64, P, P, P, P, P, P]
    assert lib.i8mm_zeropoint_matmul(*args, None, None, 4, 64, 64, P, None) == -1
    assert lib.i8mm_zeropoint_matmul(*args, P, MIS, 4, 64, 64, P, None) == -1
    assert lib.i8mm_zeropoint_matmul(*args, P, None, 4, 65536, 32768, P, None) == -1


def test_calibration_rejects():
    """The MFMA calibration validates its pointers and counts before any
    device call."""
    lib = _lib()
    assert lib.i8mm_calib_mfma_i8(None, 1, 1, P, None) == -1
    assert lib.i8mm_calib_mfma_i8(P, 1, 1, MIS, None) == -1
    assert lib.i8mm_calib_mfma_i8(P, 0, 1, P, None) == -1
    assert lib.i8mm_calib_mfma_i8(P, (1 << 20) + 1, 1, P, None) == -1
    assert lib.i8mm_calib_mfma_i8(P, 1, 0, P, None) == -1
    assert lib.i8mm_calib_mfma_i8(P, 1, (1 << 24) + 1, P, None) == -1
