"""GPU parity of the QuEST forward quantizer, the re-quantizer of saved MXFP4
operands, the mask + inverse-RHT correction and the QuEST linear layer
(forward and backward in the forward-rotated basis), against the oracle."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import mx, quest, rng

from gpu_util import assert_bytes_equal, cpu, dev_bf16, edge_case_tensor, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-5
CLIP = fq.QUEST_CLIP


def _check_quest(bits, mask, clip):
    codes, sc, mk = quest.quest_quantize(host_f32(bits), mask, clip)
    out, gm = fq.quest_quantize(dev_bf16(bits), clip=clip, mask=mask)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(out.scales), sc, "quest scales")
    assert_bytes_equal(cpu(out.codes), codes, "quest codes")
    assert_bytes_equal(cpu(gm), mk, "quest mask")


@pytest.mark.parametrize("shape", [(32, 32), (64, 256), (96, 1056), (352, 160)])
@pytest.mark.parametrize("seed", [0, 9])
def test_quest_bit_exact(shape, seed):
    log("quest", shape, seed)
    _check_quest(synth.normal_with_outliers(shape, seed, 0), rng.sign_mask(seed, 0), CLIP)


@pytest.mark.parametrize("clip", [1.0, 1.5, 4.0, 8.0, 100.0])
def test_quest_clip_values(clip):
    log("quest clip", clip)
    _check_quest(synth.normal_and_student_t((128, 512), 2, 1), rng.sign_mask(2, 0), clip)


@pytest.mark.parametrize("clip", [8.0, 1e3, 3.0e38])
def test_quest_scale_saturates(clip):
    """Thresholds beyond the E8M0 range encode as 254, on both sides."""
    log("quest huge threshold", clip)
    rs = np.random.default_rng(15)
    x = (rs.standard_normal((64, 256)) * 1e36).astype(np.float32)
    _check_quest(synth.f32_to_bf16_bits(x), rng.sign_mask(15, 0), clip)


def test_quest_edge_cases():
    log("quest edge cases")
    _check_quest(edge_case_tensor(128, 256, 3), rng.sign_mask(3, 0), CLIP)
    _check_quest(edge_case_tensor(128, 256, 4), 0, CLIP)
    x = np.zeros((32, 96), np.float32)
    x[1, :32] = -0.0
    x[2, 32] = 3.0                    # constant rotated group (sigma = 0)
    x[3, 40] = -1e-40                 # subnormal single value
    rs = np.random.default_rng(5)
    x[4:] = (rs.standard_normal((28, 96)) * np.exp(rs.uniform(-40, 40, (28, 1)))).astype(np.float32)
    _check_quest(synth.f32_to_bf16_bits(x), 0, CLIP)
    _check_quest(synth.f32_to_bf16_bits(x), rng.sign_mask(7, 0), 2.0)


def _random_mx(rows, cols, seed, lo=100, hi=150):
    rs = np.random.default_rng(seed)
    codes = rs.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rs.integers(lo, hi, (rows, cols // 32), dtype=np.uint8)
    return codes, scales


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("shape", [(32, 32), (128, 64), (96, 224), (256, 352)])
@pytest.mark.parametrize("rounding", [fq.SR, fq.RTN])
def test_requantize_bit_exact(shape, rounding):
    rows, cols = shape
    log("requant", shape, rounding)
    codes, scales = _random_mx(rows, cols, rows + cols)
    m = rng.sign_mask(4, 1)
    want_c, want_s = quest.requantize(codes, scales, m, seed=4, stream=2, rounding=rounding)
    got = fq.requantize(fq.MXTensor(_dev(codes), _dev(scales)), rounding=rounding, mask=m, seed=4,
                        rng_stream=2)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(got.scales), want_s, "requant scales")
    assert_bytes_equal(cpu(got.codes), want_c, "requant codes")


def test_requantize_special_scales():
    """Scale bytes 0 (subnormal values), 0xFF (NaN groups) and 253/254 (values
    beyond the fp32 range: inf groups) go through the same rules."""
    log("requant special scales")
    codes, scales = _random_mx(128, 96, 11)
    scales[3, 0] = 0
    scales[5, 1] = 0xFF
    scales[7, 2] = 254
    scales[9, 0] = 253
    scales[10:20, 1] = 1
    codes[12, :] = 0x88              # negative zeros
    m = rng.sign_mask(1, 2)
    want_c, want_s = quest.requantize(codes, scales, m, seed=1, stream=4)
    got = fq.requantize(fq.MXTensor(_dev(codes), _dev(scales)), mask=m, seed=1, rng_stream=4)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(got.scales), want_s, "requant scales")
    assert_bytes_equal(cpu(got.codes), want_c, "requant codes")


@pytest.mark.parametrize("shape,ldc", [((32, 32), 32), ((64, 96), 100), ((160, 1024), 1024)])
def test_unmask_inverse_hadamard(shape, ldc):
    rows, cols = shape
    log("unmask irht", shape, ldc)
    rs = np.random.default_rng(rows)
    c = rs.standard_normal((rows, ldc)).astype(np.float32)
    bits = rs.random((rows, cols)) < 0.1
    mk = np.packbits(bits, axis=1, bitorder="little")
    m = rng.sign_mask(6, 0)
    want = quest.unmask_inverse_rht(c[:, :cols], mk, m)
    t = _dev(c)
    fq.unmask_inverse_hadamard(t[:, :cols] if ldc == cols else t.as_strided((rows, cols), (ldc, 1)),
                               _dev(mk), mask=m)
    torch.cuda.synchronize()
    got = cpu(t)
    assert rel_fro(got[:, :cols], want) <= 1e-6
    assert np.max(np.abs(got[:, :cols] - want)) <= 1e-5 * np.max(np.abs(want))
    assert np.array_equal(got[:, cols:], c[:, cols:])       # padding untouched


def _oracle_layer(xf, wf, dyf, seed, clip):
    y, ctx = quest.linear_fwd(xf, wf, seed=seed, clip=clip)
    dx, dw = quest.linear_bwd(dyf, ctx)
    return y, ctx, dx, dw


@pytest.mark.parametrize("m,n,k", [(64, 96, 128), (256, 384, 160), (128, 256, 512)])
def test_quest_linear_small(m, n, k):
    log("quest linear", m, n, k)
    xb = synth.normal_with_outliers((m, k), 6, 0)
    wb = synth.normal((n, k), 0.02, 6, 1)
    dyb = synth.normal((m, n), 1e-3, 6, 2)
    seed = 13
    y, ctx = fq.quest_linear_fwd(dev_bf16(xb), dev_bf16(wb), seed=seed)
    dx, dw = fq.quest_linear_bwd(dev_bf16(dyb), ctx)
    torch.cuda.synchronize()
    ry, rctx, rdx, rdw = _oracle_layer(host_f32(xb), host_f32(wb), host_f32(dyb), seed, CLIP)
    assert_bytes_equal(cpu(ctx.xq.codes), rctx["xq"][0], "X_q codes")
    assert_bytes_equal(cpu(ctx.xq.scales), rctx["xq"][1], "X_q scales")
    assert_bytes_equal(cpu(ctx.wq.codes), rctx["wq"][0], "W_q codes")
    assert_bytes_equal(cpu(ctx.x_mask), rctx["mx"], "M_x")
    assert_bytes_equal(cpu(ctx.w_mask), rctx["mw"], "M_w")
    e = (rel_fro(cpu(y), ry), rel_fro(cpu(dx), rdx), rel_fro(cpu(dw), rdw))
    log("  rel err y %.2e dx %.2e dw %.2e" % e)
    assert max(e) <= TOL


def test_quest_linear_bwd_unbiased_on_gpu():
    """Mean over seeds of (dX_s - E[dX | forward s]) -> 0 like 1/sqrt(B)."""
    m, n, k = 64, 64, 64
    xb = synth.normal((m, k), 1.0, 7, 0)
    wb = synth.normal((n, k), 1.0, 7, 1)
    dyb = synth.normal((m, n), 1.0, 7, 2)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    xf, wf, dyf = host_f32(xb), host_f32(wb), host_f32(dyb)
    devs, one = [], None
    for s in range(96):
        _, ctx = fq.quest_linear_fwd(x, w, seed=s)
        dx, _ = fq.quest_linear_bwd(dy, ctx)
        _, rctx = quest.linear_fwd(xf, wf, seed=s, clip=CLIP)
        ex, _ = quest.expected_grads(dyf, rctx)
        d = cpu(dx) - ex
        devs.append(d)
        if one is None:
            one = np.linalg.norm(d)
    mean = np.linalg.norm(np.mean(devs, axis=0))
    log("  single %.3e mean of 96 %.3e" % (one, mean))
    assert mean < one / 5


@pytest.mark.timeout(600)
def test_quest_linear_full_size_sampled():
    """M=8192, N=K=4096 (the Quartet layer): sampled rows of X_q, M_x, Y, dX and
    dW, and whole 32-groups along K, against the oracle on those rows/groups
    (QuEST groups, masks and RNG indices are independent of the rest)."""
    d = synth.quartet_linear(0)
    xb, wb, dyb = d["x"], d["w"], d["dy"]
    m, k = xb.shape
    n = wb.shape[0]
    seed = 0
    log("quest linear full-size", m, n, k)
    y, ctx = fq.quest_linear_fwd(dev_bf16(xb), dev_bf16(wb), seed=seed)
    dx, dw = fq.quest_linear_bwd(dev_bf16(dyb), ctx)
    torch.cuda.synchronize()
    y, dx, dw = cpu(y), cpu(dx), cpu(dw)
    xq_c, xq_s, xm = cpu(ctx.xq.codes), cpu(ctx.xq.scales), cpu(ctx.x_mask)
    wm = cpu(ctx.w_mask)
    xf, wf, dyf = host_f32(xb), host_f32(wb), host_f32(dyb)
    g0, g1, g2 = (rng.sign_mask(seed, i) for i in range(3))
    rs = np.random.default_rng(77)
    ri = np.sort(rs.choice(m, 16, replace=False))
    cj = np.sort(rs.choice(n, 16, replace=False))
    gk = np.sort(rs.choice(k // 32, 3, replace=False))
    ck = (gk[:, None] * 32 + np.arange(32)[None, :]).ravel()
    mb = (gk[:, None] * 4 + np.arange(4)[None, :]).ravel()           # mask bytes of those groups
    # forward: rows ri of X_q / M_x, all of W_q on groups gk, Y[ri] on all columns
    rxc, rxs, rxm = quest.quest_quantize(xf[ri], g0, CLIP)
    assert_bytes_equal(xq_c[ri], rxc, "X_q codes (rows)")
    assert_bytes_equal(xq_s[ri], rxs, "X_q scales (rows)")
    assert_bytes_equal(xm[ri], rxm, "M_x (rows)")
    rwc, rws, rwm = quest.quest_quantize(wf, g0, CLIP)
    assert_bytes_equal(cpu(ctx.wq.codes), rwc, "W_q codes")
    assert_bytes_equal(wm, rwm, "M_w")
    ey = rel_fro(y[ri], mx.gemm(rxc, rxs, rwc, rws))
    # dX rows ri, groups gk: Q(dY)[ri] . Q(W_q^T)[ck]^T, mask, inverse RHT
    dyq = mx.quantize(dyf[ri], rounding=mx.SR, sign_mask=g1, seed=seed, stream=1, row_ids=ri)
    wdq = quest.dequantize32(rwc, rws)[:, ck]                         # [n, 96]
    wt = mx.quantize(np.ascontiguousarray(wdq.T), rounding=mx.SR, sign_mask=g1, seed=seed,
                     stream=2, row_ids=ck)
    rdx = quest.unmask_inverse_rht(mx.gemm(*dyq, *wt, alpha=mx.ALPHA_BWD), rxm[:, mb], g0)
    edx = rel_fro(dx[np.ix_(ri, ck)], rdx)
    # dW rows cj, groups gk: Q(dY^T)[cj] . Q(X_q^T)[ck]^T
    dyt = mx.quantize(np.ascontiguousarray(dyf.T[cj]), rounding=mx.SR, sign_mask=g2, seed=seed,
                      stream=3, row_ids=cj)
    xcol_c, xcol_s, _ = quest.quest_quantize(np.ascontiguousarray(xf[:, ck]), g0, CLIP)
    xdq = quest.dequantize32(xcol_c, xcol_s)                           # [m, 96]
    xt = mx.quantize(np.ascontiguousarray(xdq.T), rounding=mx.SR, sign_mask=g2, seed=seed,
                     stream=4, row_ids=ck)
    rdw = quest.unmask_inverse_rht(mx.gemm(*dyt, *xt, alpha=mx.ALPHA_BWD), rwm[cj][:, mb], g0)
    edw = rel_fro(dw[np.ix_(cj, ck)], rdw)
    log("  sampled rel err y %.2e dx %.2e dw %.2e" % (ey, edx, edw))
    assert ey <= TOL and edx <= TOL and edw <= TOL


@pytest.mark.parametrize("m,n,k,ldc", [(256, 256, 128, 256), (352, 160, 96, 160), (96, 544, 256, 576)])
def test_gemm_unmask_irht_fused(m, n, k, ldc):
    """The GEMM with the mask + inverse-RHT epilogue equals fp4mx_gemm followed
    by fp4mx_unmask_inverse_hadamard bit for bit, and the oracle within 1e-5."""
    log("gemm unmask irht", m, n, k, ldc)
    rs = np.random.default_rng(m + n)
    a = mx.quantize(host_f32(synth.normal((m, k), 1.0, 9, 0)), rounding=mx.SR, sign_mask=3, seed=2, stream=1)
    b = mx.quantize(host_f32(synth.normal((n, k), 1.0, 9, 1)), rounding=mx.SR, sign_mask=3, seed=2, stream=2)
    bits = rs.random((m, n)) < 0.05
    mk = np.packbits(bits, axis=1, bitorder="little")
    sm = rng.sign_mask(9, 0)
    A = fq.MXTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda())
    B = fq.MXTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda())
    dmk = torch.from_numpy(mk).cuda()
    c1 = torch.full((m, ldc), 7.0, dtype=torch.float32, device="cuda")
    fq.gemm_unmask_irht(A, B, dmk, alpha=16 / 9, mask=sm, out=c1[:, :n])
    c2 = torch.full((m, ldc), 7.0, dtype=torch.float32, device="cuda")
    fq.gemm(A, B, alpha=16 / 9, out=c2[:, :n])
    fq.unmask_inverse_hadamard(c2[:, :n], dmk, mask=sm)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    want = quest.unmask_inverse_rht(mx.gemm(*a, *b, alpha=mx.ALPHA_BWD), mk, sm)
    got = cpu(c1)
    assert rel_fro(got[:, :n], want) <= TOL
    assert np.all(got[:, n:] == 7.0)                     # padding columns untouched
