"""The one-call forwards' error path, driven from the host: the test hook
makes a forward's product launch report a failure without launching, so no
kernel faults or hangs. The call must return I8MM_ELAUNCH, the workspace
accumulator must be zero again once the stream has run (one more launch
clears it), and the next forward on the same workspace must be correct."""

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
import oracle.variants  # noqa: F401
from gpu_util import DEV, H, T, check_C, say
from int8_quantized_matmul_amd import _native
from workloads import random_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scheme", ["vector", "tensor", "zeropoint"])
@pytest.mark.parametrize("s", [8, 300])
def test_failed_product_launch_leaves_workspace_valid(scheme, s):
    h, o = 1024, 256
    inp = random_case(900 + s, s, h, o, 5, row_frac=0.5)
    X, W = inp["X"], inp["W"]
    Xd, Wd = T(X), T(W)
    qw = i8.quantize_weights(Wd, scheme)
    ws = i8.forward_workspace(s, h, DEV, zeropoint=True)

    def run():
        if scheme == "zeropoint":
            return i8.forward_zeropoint(Xd, qw, Wd, 6.0, workspace=ws)
        if scheme == "tensor":
            return i8.forward_tensorwise(Xd, qw[0], qw[1], Wd, 6.0, workspace=ws)
        return i8.forward(Xd, qw[0], qw[1], Wd, 6.0, workspace=ws)

    lib = _native.load()
    say(f"  launch: {scheme} forward s={s} with the product launch failed by the hook")
    lib.i8mm_test_fail_product_launches(1)
    try:
        with pytest.raises(i8.I8MMError, match=r"status -3"):
            run()
    finally:
        lib.i8mm_test_fail_product_launches(0)
    torch.cuda.synchronize()
    assert not H(ws[: i8.ACC_BYTES]).any(), "accumulator left non-zero after the failed call"
    say(f"  launch: {scheme} forward s={s} again")
    C = run()
    torch.cuda.synchronize()
    assert not H(ws[: i8.ACC_BYTES]).any()
    check_C(C, oracle.variants.variant_forward(X, W, scheme, 6.0) if scheme != "vector"
            else oracle.forward(X, W, 6.0)["C"])
