"""The entry points under HIP graph capture (torch.cuda.graph): no call
allocates or uses a memset node (counters are zeroed by kernels), so a
captured step replays correctly.  Each graph is replayed several times with
eager calls and synchronisations in between, and every replay must equal the
eager result bit for bit."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth

from gpu_util import dev_bf16, log

pytestmark = pytest.mark.gpu

M = N = K = 256


@pytest.fixture(scope="module")
def data():
    return (dev_bf16(synth.normal_with_outliers((M, K), 8, 0)), dev_bf16(synth.normal((N, K), 0.02, 8, 1)),
            dev_bf16(synth.normal((M, N), 1e-3, 8, 2)))


def _check_graph(fn, what):
    log("graph", what)
    want = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = fn()
    for rep in range(3):
        for t in got:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), (what, rep)
        fn()                                   # eager work between replays
        torch.cuda.synchronize()


def test_graph_mx_linear(data):
    x, w, dy = data

    def step():
        y, ctx = fq.linear_fwd(x, w, seed=3)
        dx, dw = fq.linear_bwd(dy, ctx)
        return y, dx, dw, ctx.xt.codes, ctx.wt.scales
    _check_graph(step, "mx linear fwd+bwd")


def test_graph_quest_linear(data):
    x, w, dy = data

    def step():
        y, ctx = fq.quest_linear_fwd(x, w, seed=4)
        dx, dw = fq.quest_linear_bwd(dy, ctx)
        return y, dx, dw
    _check_graph(step, "quest linear fwd+bwd")


def test_graph_nvfp4(data):
    x, w, dy = data

    def step():
        y = fq.nv_linear_fwd(x, w)
        q = fq.nv_quantize46(x)
        e = fq.nv_msedn_quantize(dy, axis=fq.COL, seed=2, gemm_id=1, stream=5)
        s = fq.nv_sr_quantize(dy, seed=2, stream=1)
        dx, dw = fq.nv_linear_bwd(dy, x, w, seed=5)
        return y, q.codes, q.scales, q.tensor_scale, e.codes, e.scales, e.tensor_scale, s.codes, dx, dw
    _check_graph(step, "nvfp4 forward, quantizers and backward")
