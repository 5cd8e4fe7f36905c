"""fp8_linear_noalloc (the library's static device scratch, no workspace
argument) against fp8_linear (caller workspace), both through the C-ABI:
two calls in a row, the second with a smaller input. Codes and scales must
be bit-identical; y bit-identical where fp8_linear's split-K plan fits the
scratch, else within the output tolerance of fp8_linear's y."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_y_close, dev_bf16, ensure_built, host_bf16_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ensure_built()


def noalloc(L, x, qw, sw):
    M, K = x.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.fp8_linear_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(qw.data_ptr()),
                              ctypes.c_void_p(sw.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                              M, N, K, ctypes.c_void_p(qx.data_ptr()),
                              ctypes.c_void_p(sx.data_ptr()), 0, st)
    assert rc == 0, f"fp8_linear_noalloc: status {rc}"
    return y, qx, sx


# (M, N, K, fp8_linear's plan fits the scratch): the 70B qkv at 64 tokens
# needs 21 MB of partials (capped to fewer slices here); the 70B down at 64
# tokens exactly 16 MiB; then smaller calls
CALLS = [(64, 10240, 8192, False), (64, 8192, 28672, True), (1, 1024, 16384, True),
         (20, 100, 65536, True), (3, 256, 4096, True)]


def test_noalloc_matches_linear(F):
    L = F.lib()
    for i, (M, N, K, fits) in enumerate(CALLS):
        say(f"noalloc call {i}: {M}x{N}x{K}")
        x = dev_bf16(synth.activations(M, K, 70 + i, 80 + i))
        qw, sw = F.fp8_quant_act(dev_bf16(synth.weights(N, K, 90 + i)))
        y_na, qx_na, sx_na = noalloc(L, x, qw, sw)
        y_ref, qx_ref, sx_ref = F.fp8_linear(x, qw, sw)
        torch.cuda.synchronize()
        assert torch.equal(qx_na, qx_ref), f"call {i}: codes"
        assert torch.equal(sx_na.view(torch.int32), sx_ref.view(torch.int32)), f"call {i}: scales"
        if fits:
            assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), f"call {i}: y"
        else:
            assert_y_close(host_bf16_f64(y_na), host_bf16_f64(y_ref), f"call {i} y")
    # the static scratch is left reusable: repeat the first call
    M, N, K, _ = CALLS[0]
    x = dev_bf16(synth.activations(M, K, 70, 80))
    qw, sw = F.fp8_quant_act(dev_bf16(synth.weights(N, K, 90)))
    y1, _, _ = noalloc(L, x, qw, sw)
    y2, _, _ = noalloc(L, x, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "repeat"


# split-K decode shapes (the tile counters must be back at zero for the next
# replay), the split quantizer of long rows, and a prefill shape
GRAPH_CASES = [(20, 100, 65536), (64, 8192, 28672), (8, 10240, 8192), (256, 1024, 4096)]


def test_noalloc_graph_replay(F):
    """fp8_linear_noalloc captured in a HIP graph, as the callers it is for
    use it: the captured calls replayed 5 times, with eager work (the outputs
    cleared) and synchronizations between replays; every replay bit-identical
    to the eager calls."""
    L = F.lib()
    bufs = []
    for i, (M, N, K) in enumerate(GRAPH_CASES):
        x = dev_bf16(synth.activations(M, K, 170 + i, 180 + i))
        qw, sw = F.fp8_quant_act(dev_bf16(synth.weights(N, K, 190 + i)))
        outs = (torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                torch.empty((M,), dtype=torch.float32, device="cuda"))
        bufs.append((x, qw, sw) + outs)

    def call_all():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for x, qw, sw, y, qx, sx in bufs:
            M, K = x.shape
            rc = L.fp8_linear_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(qw.data_ptr()),
                                      ctypes.c_void_p(sw.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                      M, qw.shape[0], K, ctypes.c_void_p(qx.data_ptr()),
                                      ctypes.c_void_p(sx.data_ptr()), 0, st)
            assert rc == 0, f"fp8_linear_noalloc: status {rc}"

    say("noalloc graph: eager calls")
    call_all()          # eager reference; also sets up every launch path
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in b[3:]) for b in bufs]
    say("noalloc graph: capture")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        call_all()
    torch.cuda.synchronize()
    for r in range(5):
        for b in bufs:
            for t in b[3:]:
                t.zero_()
        torch.cuda.synchronize()
        say(f"noalloc graph: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for i, (b, rf) in enumerate(zip(bufs, ref)):
            y, qx, sx = b[3:]
            assert torch.equal(qx, rf[1]), f"replay {r}, case {i}: codes"
            assert torch.equal(sx.view(torch.int32), rf[2].view(torch.int32)), f"replay {r}, case {i}: scales"
            assert torch.equal(y.view(torch.int16), rf[0].view(torch.int16)), f"replay {r}, case {i}: y"
