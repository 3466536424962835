"""GPU parity of the fully-FP4 linear layer (forward + backward) against the oracle.

Small shapes are compared in full; the Quartet-style (8192 x 4096 x 4096) and
Llama-3-8B FFN-up (8192 x 4096 -> 14336) workloads are checked at full size,
with the entry points the benchmark times, on sampled outputs whose oracle
operands are computed row by row."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import mx, rng

from gpu_util import assert_bytes_equal, assert_gemm_close, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _run(xb, wb, dyb, seed):
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    y, ctx = fq.linear_fwd(x, w, seed=seed)
    dx, dw = fq.linear_bwd(dy, ctx)
    torch.cuda.synchronize()
    return y, ctx, dx, dw


def test_tiny_forward_workload():
    """X 64x128, W 128x128, N(0,1) with 1% x20 outliers, seeded RHT, RTN, Y fp32."""
    d = synth.tiny_linear(0)
    for seed in (0, 9):
        y, _ = fq.linear_fwd(dev_bf16(d["x"]), dev_bf16(d["w"]), seed=seed, want_ctx=False)
        want, _ = mx.linear_fwd(host_f32(d["x"]), host_f32(d["w"]), seed, want_ctx=False)
        err = rel_fro(cpu(y), want)
        log("tiny fwd seed", seed, "rel err", err)
        assert err <= TOL


@pytest.mark.parametrize("m,n,k", [(128, 96, 160), (64, 64, 64), (256, 384, 512), (96, 32, 224)])
def test_forward_backward_small(m, n, k):
    log("linear", m, n, k)
    xb = synth.normal((m, k), 1.0, 3, 0)
    wb = synth.normal((n, k), 0.02, 3, 1)
    dyb = synth.normal((m, n), 1e-3, 3, 2)
    seed = 17
    y, ctx, dx, dw = _run(xb, wb, dyb, seed)
    xf, wf, dyf = host_f32(xb), host_f32(wb), host_f32(dyb)
    ry, rctx = mx.linear_fwd(xf, wf, seed)
    assert_bytes_equal(cpu(ctx.xt.codes), rctx["xt"][0], "ctx xt codes")
    assert_bytes_equal(cpu(ctx.xt.scales), rctx["xt"][1], "ctx xt scales")
    assert_bytes_equal(cpu(ctx.wt.codes), rctx["wt"][0], "ctx wt codes")
    assert_bytes_equal(cpu(ctx.wt.scales), rctx["wt"][1], "ctx wt scales")
    # the layer's GEMM operands, each from the oracle's quantizer
    g0, g1, g2 = (rng.sign_mask(seed, i) for i in range(3))
    deq = lambda q: mx.dequantize(*q)
    qx = mx.quantize(xf, rounding=mx.RTN, sign_mask=g0)
    qw = mx.quantize(wf, rounding=mx.RTN, sign_mask=g0)
    qdy = mx.quantize(dyf, rounding=mx.SR, sign_mask=g1, seed=seed, stream=1)
    qdyt = mx.quantize(dyf, rounding=mx.SR, axis=mx.COL, sign_mask=g2, seed=seed, stream=3)
    assert_gemm_close(cpu(y), deq(qx), deq(qw), 1.0, "y")
    assert_gemm_close(cpu(dx), deq(qdy), deq(rctx["wt"]), mx.ALPHA_BWD, "dx")
    assert_gemm_close(cpu(dw), deq(qdyt), deq(rctx["xt"]), mx.ALPHA_BWD, "dw")
    rdx, rdw = mx.linear_bwd(dyf, rctx)
    for name, got, want in (("y", y, ry), ("dx", dx, rdx), ("dw", dw, rdw)):
        err = rel_fro(cpu(got), want)
        log("  ", name, "rel err", err)
        assert err <= TOL


def test_backward_unbiased_on_gpu():
    """Mean of B independent GPU backward estimates -> exact gradient, error ~ 1/B."""
    m, n, k = 64, 64, 128
    xb = synth.normal((m, k), 1.0, 4, 0)
    wb = synth.normal((n, k), 1.0, 4, 1)
    dyb = synth.normal((m, n), 1.0, 4, 2)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    ex_dx = host_f32(dyb).astype(np.float64) @ host_f32(wb).astype(np.float64)
    ex_dw = host_f32(dyb).T.astype(np.float64) @ host_f32(xb).astype(np.float64)
    dxs, dws = [], []
    for seed in range(256):
        _, ctx = fq.linear_fwd(x, w, seed=seed)
        dx, dw = fq.linear_bwd(dy, ctx)
        dxs.append(cpu(dx))
        dws.append(cpu(dw))
    for ests, ex in ((np.array(dxs), ex_dx), (np.array(dws), ex_dw)):
        def mse(B):
            mm = ests[: (len(ests) // B) * B].reshape(-1, B, *ex.shape).mean(axis=1)
            return np.mean((mm - ex) ** 2)
        e1, e16, e64 = mse(1), mse(16), mse(64)
        log("  1/B mse", e1, e16, e64)
        assert e16 < e1 / 8 and e64 < e1 / 30


def _sampled_full_size(d, seed, nsamp=48):
    x, w, dy = d["x"], d["w"], d["dy"]
    m, k = x.shape
    n = w.shape[0]
    log("full-size linear", m, n, k)
    y, ctx, dx, dw = _run(x, w, dy, seed)
    rs = np.random.default_rng(123)
    ri = np.sort(rs.choice(m, nsamp, replace=False))   # rows of Y / dX
    cj = np.sort(rs.choice(n, nsamp, replace=False))   # cols of Y / rows of dW
    ck = np.sort(rs.choice(k, nsamp, replace=False))   # cols of dX / dW
    xf, wf, dyf = host_f32(x), host_f32(w), host_f32(dy)
    g0, g1, g2 = (rng.sign_mask(seed, i) for i in range(3))
    # Y[ri, cj]: rows of Q_RTN(RHT_K X) and Q_RTN(RHT_K W)
    qx = mx.quantize(xf[ri], rounding=mx.RTN, sign_mask=g0)
    qw = mx.quantize(wf[cj], rounding=mx.RTN, sign_mask=g0)
    ey = rel_fro(cpu(y)[np.ix_(ri, cj)], mx.gemm(*qx, *qw))
    # context rows: W^T rows ck (W columns, SR along N, stream 2) and X^T rows ck
    wt = mx.quantize(wf[:, ck], rounding=mx.SR, axis=mx.COL, sign_mask=g1, seed=seed, stream=2, row_ids=ck)
    xt = mx.quantize(xf[:, ck], rounding=mx.SR, axis=mx.COL, sign_mask=g2, seed=seed, stream=4, row_ids=ck)
    assert_bytes_equal(cpu(ctx.wt.codes)[ck], wt[0], "ctx wt codes (sampled rows)")
    assert_bytes_equal(cpu(ctx.wt.scales)[ck], wt[1], "ctx wt scales (sampled rows)")
    assert_bytes_equal(cpu(ctx.xt.codes)[ck], xt[0], "ctx xt codes (sampled rows)")
    assert_bytes_equal(cpu(ctx.xt.scales)[ck], xt[1], "ctx xt scales (sampled rows)")
    # dX[ri, ck] = 16/9 Q_SR(RHT_N dY)[ri] . W^T[ck]
    qdy = mx.quantize(dyf[ri], rounding=mx.SR, sign_mask=g1, seed=seed, stream=1, row_ids=ri)
    edx = rel_fro(cpu(dx)[np.ix_(ri, ck)], mx.gemm(*qdy, *wt, alpha=16 / 9))
    # dW[cj, ck] = 16/9 Q_SR(RHT_M dY^T)[cj] . X^T[ck]
    qdyt = mx.quantize(dyf[:, cj], rounding=mx.SR, axis=mx.COL, sign_mask=g2, seed=seed, stream=3,
                       row_ids=cj)
    edw = rel_fro(cpu(dw)[np.ix_(cj, ck)], mx.gemm(*qdyt, *xt, alpha=16 / 9))
    log("  sampled rel err y %.2e dx %.2e dw %.2e" % (ey, edx, edw))
    assert ey <= TOL and edx <= TOL and edw <= TOL


def test_quartet_workload_full_size():
    _sampled_full_size(synth.quartet_linear(0), seed=0)


def test_llama_ffn_up_workload_full_size():
    _sampled_full_size(synth.llama_ffn_up(0), seed=0)


@pytest.mark.parametrize("m,n,k", [(128, 96, 160), (256, 384, 512)])
def test_bf16_output_entry_points(m, n, k):
    """fp4mx_linear_fwd_bf16 / _bwd_bf16 write bf16_RNE of what the fp32
    entry points write, bit for bit, and share their context bytes."""
    log("linear bf16 out", m, n, k)
    xb = synth.normal_with_outliers((m, k), 5, 0)
    wb = synth.normal((n, k), 0.02, 5, 1)
    dyb = synth.normal((m, n), 1e-3, 5, 2)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    y32, c32 = fq.linear_fwd(x, w, seed=8)
    dx32, dw32 = fq.linear_bwd(dy, c32)
    y16, c16 = fq.linear_fwd(x, w, seed=8, dtype=torch.bfloat16)
    dx16, dw16 = fq.linear_bwd(dy, c16, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    bits = lambda t: cpu(t.view(torch.int16)).view(np.uint16)
    for a, b in ((c16.xt, c32.xt), (c16.wt, c32.wt)):
        assert_bytes_equal(cpu(a.codes), cpu(b.codes), "ctx codes")
        assert_bytes_equal(cpu(a.scales), cpu(b.scales), "ctx scales")
    for name, got, want in (("y", y16, y32), ("dx", dx16, dx32), ("dw", dw16, dw32)):
        assert got.dtype == torch.bfloat16
        assert_bytes_equal(bits(got), synth.f32_to_bf16_bits(cpu(want)), name + " bf16")


@pytest.mark.parametrize("m,n,k", [(352, 96, 288), (96, 1056, 480), (1056, 2080, 1056)])
def test_forward_one_launch_quantizer(m, n, k):
    """fp4mx_linear_fwd quantizes X and W in one launch; its Y and context
    equal, bit for bit, the single-operand dual quantizer on each operand
    followed by fp4mx_gemm (shapes with ragged tiles and different tile
    grids for X and W)."""
    log("linear fwd one-launch quantizer", m, n, k)
    xb = synth.normal_with_outliers((m, k), 6, 0)
    wb = synth.normal((n, k), 0.02, 6, 1)
    x, w = dev_bf16(xb), dev_bf16(wb)
    seed = 23
    y, ctx = fq.linear_fwd(x, w, seed=seed)
    g0, g1, g2 = (fq.sign_mask(seed, i) for i in range(3))
    xr, xc = fq.hadamard_quantize_dual(x, fq.RTN, g0, 0, fq.SR, g2, 4, seed=seed)
    wr, wc = fq.hadamard_quantize_dual(w, fq.RTN, g0, 0, fq.SR, g1, 2, seed=seed)
    y1 = fq.gemm(xr, wr)
    torch.cuda.synchronize()
    for name, a, b in (("xt", ctx.xt, xc), ("wt", ctx.wt, wc)):
        assert_bytes_equal(cpu(a.codes), cpu(b.codes), name + " codes")
        assert_bytes_equal(cpu(a.scales), cpu(b.scales), name + " scales")
    assert torch.equal(y, y1)


def test_autograd_function():
    """FP4LinearFunction under torch.autograd: Y and both gradients are the bf16
    roundings (nearest even) of fp4mx_linear_fwd / _bwd's fp32 outputs, bit for
    bit, and the fp32 values agree with the oracle's forward and backward."""
    m, n, k, seed = 128, 96, 160, 6
    xb = synth.normal_with_outliers((m, k), 4, 0)
    wb = synth.normal((n, k), 0.02, 4, 1)
    gb = synth.normal((m, n), 1e-3, 4, 2)
    x = dev_bf16(xb).requires_grad_(True)
    w = dev_bf16(wb).requires_grad_(True)
    g = dev_bf16(gb)
    y = fq.FP4LinearFunction.apply(x, w, seed)
    y.backward(g)
    y32, ctx = fq.linear_fwd(x.detach(), w.detach(), seed=seed)
    dx32, dw32 = fq.linear_bwd(g, ctx)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16 and x.grad.dtype == torch.bfloat16
    bits = lambda t: cpu(t.detach().view(torch.int16)).view(np.uint16)
    assert np.array_equal(bits(y), synth.f32_to_bf16_bits(cpu(y32)))
    assert np.array_equal(bits(x.grad), synth.f32_to_bf16_bits(cpu(dx32)))
    assert np.array_equal(bits(w.grad), synth.f32_to_bf16_bits(cpu(dw32)))
    want_y, octx = mx.linear_fwd(host_f32(xb), host_f32(wb), seed)
    want_dx, want_dw = mx.linear_bwd(host_f32(gb), octx)
    assert rel_fro(cpu(y32), want_y) <= TOL
    assert rel_fro(cpu(dx32), want_dx) <= TOL and rel_fro(cpu(dw32), want_dw) <= TOL
