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
                                    [(64, 8192, 768, 7), (8, 2048, 256, 3)],
                                    [(8, 1024, 256, 3), (2, 512, 128, 2)]],
                         ids=["prefill then smaller", "few rows then decode", "one-launch prologue twice"])
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


def test_noalloc_graph_replays():
    """The use the entry point exists for: three allocation-free forwards (a
    prefill shape and two decode shapes, one per few-row prologue route)
    captured in one HIP graph (torch's CUDA-graph
    API over the library's stream-ordered launches) and replayed four times.
    Between replays, eager work runs: a fill of the outputs, and an eager
    allocation-free forward on other inputs that rewrites the shared scratch.
    Every replay must reproduce the workspace forward's C bit for bit."""
    cases = [(300, 1024, 512, 5), (8, 2048, 256, 3), (4, 1024, 256, 3)]
    data = []
    for k, (s, h, o, nout) in enumerate(cases):
        inp = random_case(760 + k, s, h, o, nout, row_frac=0.5)
        Xd, Wd = T(inp["X"]), T(inp["W"])
        Wq, c_w = i8.quantize_colwise_weights(Wd)
        ref = i8.forward(Xd, Wq, c_w, Wd, 6.0)
        data.append((Xd, Wd, Wq, c_w, ref, torch.empty_like(ref)))
    other = random_case(790, 512, 1024, 512, 9, row_frac=0.5)
    Xo, Wo = T(other["X"]), T(other["W"])
    Wqo, cwo = i8.quantize_colwise_weights(Wo)
    ref_o = i8.forward(Xo, Wqo, cwo, Wo, 6.0)
    Co = torch.empty_like(ref_o)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # first calls outside the capture
        for Xd, Wd, Wq, c_w, _, C in data:
            i8.forward_noalloc(Xd, Wq, c_w, Wd, 6.0, C=C)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    say("  capture: three forward_noalloc calls")
    with torch.cuda.graph(g):
        for Xd, Wd, Wq, c_w, _, C in data:
            i8.forward_noalloc(Xd, Wq, c_w, Wd, 6.0, C=C)
    torch.cuda.synchronize()
    for r in range(4):
        for *_, C in data:
            C.fill_(float("nan"))
        i8.forward_noalloc(Xo, Wqo, cwo, Wo, 6.0, C=Co)
        torch.cuda.synchronize()
        assert torch.equal(Co, ref_o), f"eager call before replay {r + 1}"
        say(f"  replay {r + 1}")
        g.replay()
        torch.cuda.synchronize()
        for k, (*_, ref, C) in enumerate(data):
            assert torch.equal(C, ref), f"replay {r + 1}: forward {k} differs from the workspace forward"
