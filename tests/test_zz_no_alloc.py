"""i8mm_forward_noalloc (the forward over the library's static device
scratch, for callers that cannot allocate) called through the C ABI and
compared with i8mm_forward on the same inputs: two calls in a row, the
second with a smaller input, each bit for bit equal to the workspace
forward's C and within 2e-3 ||C_ref||_inf of the oracle; a shape beyond
the scratch is rejected with I8MM_ESCRATCH before anything runs."""

import ctypes

import numpy as np
import pytest
import torch

import int8_quantized_matmul_amd as i8
import oracle
from gpu_util import DEV, H, T, check_C, say
from int8_quantized_matmul_amd import _native
from workloads import random_case

pytestmark = pytest.mark.gpu

I8MM_ESCRATCH = -5


def _noalloc(lib, Xd, Wq, c_w, Wd, alpha, C):
    s, h = Xd.shape
    o = C.shape[1]
    st = lib.i8mm_forward_noalloc(Xd.data_ptr(), s, h, o, alpha, Wq.data_ptr(), c_w.data_ptr(), Wd.data_ptr(), None,
                                  C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("shapes", [[(2048, 4096, 1024, 6), (300, 1024, 512, 5)],
                                    [(64, 8192, 768, 7), (8, 2048, 256, 3)]],
                         ids=["prefill then smaller", "few rows then decode"])
def test_noalloc_matches_workspace_forward(shapes):
    lib = _native.load()
    for k, (s, h, o, nout) in enumerate(shapes):
        assert lib.i8mm_forward_workspace_bytes(s, h) <= i8.NOALLOC_SCRATCH_BYTES
        inp = random_case(700 + 31 * k + s, s, h, o, nout, row_frac=0.5)
        X, W = inp["X"], inp["W"]
        Xd, Wd = T(X), T(W)
        Wq, c_w = i8.quantize_colwise_weights(Wd)
        C_ws = i8.forward(Xd, Wq, c_w, Wd, 6.0)
        C_na = torch.full((s, o), float("nan"), dtype=torch.float16, device=DEV)
        say(f"  launch: forward_noalloc call {k + 1} s={s} h={h} o={o}")
        assert _noalloc(lib, Xd, Wq, c_w, Wd, 6.0, C_na) == 0
        torch.cuda.synchronize()
        assert torch.equal(C_na, C_ws), f"call {k + 1}: noalloc C differs from the workspace forward"
        check_C(C_na, oracle.forward(X, W, 6.0)["C"])


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = _native.load()
    s, h, o = 4096, 8192, 64
    assert lib.i8mm_forward_workspace_bytes(s, h) > i8.NOALLOC_SCRATCH_BYTES
    Xd = torch.zeros((s, h), dtype=torch.float16, device=DEV)
    Wd = torch.zeros((h, o), dtype=torch.float16, device=DEV)
    Wq, c_w = i8.quantize_colwise_weights(Wd)
    C = torch.full((s, o), 7.0, dtype=torch.float16, device=DEV)
    say("  launch: forward_noalloc beyond the scratch (rejected on the host)")
    assert _noalloc(lib, Xd, Wq, c_w, Wd, 6.0, C) == I8MM_ESCRATCH
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a rejected call wrote C"
    with pytest.raises(i8.I8MMError, match=r"status -5"):
        i8.forward_noalloc(Xd, Wq, c_w, Wd, 6.0, C=C)
