"""Concurrent calls on different streams (the C ABI holds no per-call state;
each call brings its own workspace and output): one-call forwards of three
shapes (prefill, decode, small prefill) and a load-time weight conversion,
interleaved on two streams of default priority for three rounds, must give
results bit for bit equal to the same calls run one after another."""

import pytest
import torch

import int8_quantized_matmul_amd as i8
from gpu_util import DEV, T, say
from workloads import random_case

pytestmark = pytest.mark.gpu

CASES = [(300, 2048, 1024, 6), (8, 4096, 2048, 5), (1024, 1024, 768, 3)]


def test_forwards_and_conversion_on_two_streams():
    prepared = []
    for k, (s, h, o, nout) in enumerate(CASES):
        inp = random_case(1500 + k, s, h, o, nout, row_frac=0.5)
        Xd, Wd = T(inp["X"]), T(inp["W"])
        Wq, c_w = i8.quantize_colwise_weights(Wd)
        ref = i8.forward(Xd, Wq, c_w, Wd, 6.0)
        ws = i8.forward_workspace(s, h, DEV)
        prepared.append((Xd, Wd, Wq, c_w, ref, ws, torch.empty_like(ref)))
    Wn = T(random_case(1590, 1, 4096, 4096, 0)["W"])
    Wq_ref, cw_ref = i8.quantize_colwise_weights(Wn)
    Wq_n, cw_n = torch.empty_like(Wq_ref), torch.empty_like(cw_ref)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    say("  launch: three rounds of forwards on two streams, a weight conversion on the second")
    for rnd in range(3):
        for k, (Xd, Wd, Wq, c_w, _, ws, C) in enumerate(prepared):
            with torch.cuda.stream(streams[k % 2]):
                i8.forward(Xd, Wq, c_w, Wd, 6.0, workspace=ws, C=C)
        if rnd == 1:
            with torch.cuda.stream(streams[1]):
                i8.quantize_colwise_weights(Wn, Wq_n, cw_n)
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for k, (*_, ref, ws, C) in enumerate(prepared):
        assert torch.equal(C, ref), f"forward {k} on stream {k % 2} differs from the serial run"
    assert torch.equal(Wq_n, Wq_ref) and torch.equal(cw_n, cw_ref), "conversion on the second stream differs"
