"""The int8 MFMA calibration stream (i8mm_calib_mfma_i8), which the
benchmark uses for the practical ceiling of the prefill product: it runs
through the C ABI, reports the operations it performs, and is deterministic
(the same codes give the same accumulator digest on every call)."""

import pytest
import torch

import int8_quantized_matmul_amd as i8
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def test_calibration_stream_runs_and_is_deterministic():
    blocks, iters = 8, 64
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    codes = torch.randint(-127, 128, (blocks * 65536,), generator=g, dtype=torch.int8, device=DEV)
    out1 = torch.empty((blocks * 256,), dtype=torch.int32, device=DEV)
    out2 = torch.empty_like(out1)
    say(f"  launch: calib_mfma_i8 blocks={blocks} iters={iters}")
    ops = i8.calib_mfma_i8(codes, iters, out1)
    i8.calib_mfma_i8(codes, iters, out2)
    torch.cuda.synchronize()
    assert ops == blocks * 4 * 32 * iters * 65536
    assert torch.equal(out1, out2)
    assert bool((out1 != 0).any())
    with pytest.raises(ValueError):
        i8.calib_mfma_i8(codes, iters, torch.empty((100,), dtype=torch.int32, device=DEV))
