"""GPU parity of the NVFP4 backward that re-quantizes the saved forward
operands with MS-EDEN (the Quartet II graph), against the oracle."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import msedn, nvfp4, quartet2 as q2

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _nv_dev(codes, scales, g):
    return fq.NVTensor(torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(scales)).cuda(),
                       torch.tensor([np.float32(g)], dtype=torch.float32).cuda())


def _check_requant(codes, scales, g, seed, gemm_id, stream):
    words = msedn.sign_mask128(seed, gemm_id)
    rc, rs, rg, S = q2.requantize(codes, scales, g, words, seed, stream)
    out, s_gpu = fq.nv_msedn_requantize(_nv_dev(codes, scales, g), seed=seed, gemm_id=gemm_id,
                                        stream=stream, want_s=True)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == rg
    assert_bytes_equal(cpu(s_gpu).view(np.uint32), S.view(np.uint32), "EDEN S")
    assert_bytes_equal(cpu(out.codes), rc, "requant codes")
    assert_bytes_equal(cpu(out.scales), rs, "requant scales")


@pytest.mark.parametrize("shape", [(128, 32), (256, 96), (384, 160), (128, 1024)])
def test_nv_requant_of_saved_operand_bit_exact(shape):
    log("nv requant", shape)
    x = host_f32(synth.normal_with_outliers(shape, 4, 1))
    codes, scales, g = nvfp4.quantize46(x, True)
    _check_requant(codes, scales, g, 3, 1, 6)


def test_nv_requant_synthetic_bytes():
    """Arbitrary code / scale bytes and tensor scales from tiny to huge."""
    rs = np.random.default_rng(8)
    for g in (np.float32(1.0), np.float32(3.7e-3), np.float32(2.5e-38), np.float32(1.1e30)):
        log("nv requant bytes g", g)
        codes = rs.integers(0, 256, (256, 32), dtype=np.uint8)
        scales = rs.integers(0, 0x7F, (256, 4), dtype=np.uint8)        # finite E4M3 (no NaN)
        scales[5] = 0
        codes[7] = 0x88
        _check_requant(codes, scales, g, 5, 2, 8)


def _layer(m, n, k, seed):
    xb = synth.normal_with_outliers((m, k), seed, 0)
    wb = synth.normal((n, k), 0.02, seed, 1)
    dyb = synth.normal((m, n), 1e-3, seed, 2)
    return xb, wb, dyb


@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 384, 160), (128, 256, 512)])
def test_nv_linear_ctx_small(m, n, k):
    log("nv linear ctx", m, n, k)
    xb, wb, dyb = _layer(m, n, k, 5)
    y, ctx = fq.nv_linear_fwd_ctx(dev_bf16(xb), dev_bf16(wb), seed=21)
    dx, dw = fq.nv_linear_bwd_ctx(dev_bf16(dyb), ctx)
    torch.cuda.synchronize()
    ry, rctx = q2.linear_fwd(host_f32(xb), host_f32(wb))
    for got, want, nm in ((ctx.xq, rctx["xq"], "Q(X)"), (ctx.wq, rctx["wq"], "Q(W)")):
        assert_bytes_equal(cpu(got.codes), want[0], nm + " codes")
        assert_bytes_equal(cpu(got.scales), want[1], nm + " scales")
        assert cpu(got.tensor_scale)[0] == want[2]
    rdx, rdw = q2.linear_bwd(host_f32(dyb), rctx, 21)
    e = (rel_fro(cpu(y), ry), rel_fro(cpu(dx), rdx), rel_fro(cpu(dw), rdw))
    log("  rel err y %.2e dx %.2e dw %.2e" % e)
    assert max(e) <= TOL


def test_nv_linear_bwd_ctx_unbiased_on_gpu():
    m, n, k = 128, 128, 64
    xb = synth.normal((m, k), 1.0, 6, 0)
    wb = synth.normal((n, k), 1.0, 6, 1)
    dyb = synth.normal((m, n), 1.0, 6, 2)
    y, ctx = fq.nv_linear_fwd_ctx(dev_bf16(xb), dev_bf16(wb), seed=0)
    _, rctx = q2.linear_fwd(host_f32(xb), host_f32(wb))
    ex_dx, ex_dw = q2.expected_grads(host_f32(dyb), rctx)
    dy = dev_bf16(dyb)
    dxs, dws = [], []
    for seed in range(256):
        ctx.seed = seed
        dx, dw = fq.nv_linear_bwd_ctx(dy, ctx)
        dxs.append(cpu(dx))
        dws.append(cpu(dw))
    for ests, ex in ((np.array(dxs), ex_dx), (np.array(dws), ex_dw)):
        def mse(B):
            mm = ests[: (len(ests) // B) * B].reshape(-1, B, *ex.shape).mean(axis=1)
            return np.mean((mm - ex) ** 2)
        e1, e16, e64 = mse(1), mse(16), mse(64)
        log("  1/B mse", e1, e16, e64)
        assert e16 < e1 / 8 and e64 < e1 / 25


@pytest.mark.timeout(900)
def test_nv_linear_ctx_full_size_sampled():
    """M=8192, N=K=4096: Q(X), Q(W) in full, then sampled rows of dX and dW
    against oracle operands built row by row with the full tensors' ranges."""
    d = synth.quartet_linear(0)
    xb, wb, dyb = d["x"], d["w"], d["dy"]
    m, k = xb.shape
    n = wb.shape[0]
    seed = 0
    log("nv linear ctx full-size", m, n, k)
    y, ctx = fq.nv_linear_fwd_ctx(dev_bf16(xb), dev_bf16(wb), seed=seed)
    dx, dw = fq.nv_linear_bwd_ctx(dev_bf16(dyb), ctx)
    torch.cuda.synchronize()
    dx, dw = cpu(dx), cpu(dw)
    xf, wf, dyf = host_f32(xb), host_f32(wb), host_f32(dyb)
    xq = nvfp4.quantize46(xf, True)
    wq = nvfp4.quantize46(wf, True)
    assert_bytes_equal(cpu(ctx.xq.codes), xq[0], "Q(X) codes")
    assert_bytes_equal(cpu(ctx.wq.scales), wq[1], "Q(W) scales")
    w1, w2 = msedn.sign_mask128(seed, 1), msedn.sign_mask128(seed, 2)
    rs = np.random.default_rng(99)
    ri = np.sort(rs.choice(m, 16, replace=False))
    cj = np.sort(rs.choice(n, 16, replace=False))
    ck = np.sort(rs.choice(k, 16, replace=False))
    k_a = msedn.msedn_range_exponent(dyf, w1)
    a = msedn.msedn_quantize(dyf[ri], w1, seed=seed, stream=5, row_ids=ri, k=k_a)[:3]
    k_b = q2.requant_range_exponent(*wq, w1)
    b = q2.requantize(*wq, w1, seed, 6, row_ids=ck, k=k_b)[:3]
    edx = rel_fro(dx[np.ix_(ri, ck)], nvfp4.gemm_fp8_staged(*a, *b))
    dyt = np.ascontiguousarray(dyf.T)
    k_c = msedn.msedn_range_exponent(dyt, w2)
    c = msedn.msedn_quantize(dyt[cj], w2, seed=seed, stream=7, row_ids=cj, k=k_c)[:3]
    k_d = q2.requant_range_exponent(*xq, w2)
    dd = q2.requantize(*xq, w2, seed, 8, row_ids=ck, k=k_d)[:3]
    edw = rel_fro(dw[np.ix_(cj, ck)], nvfp4.gemm_fp8_staged(*c, *dd))
    log("  sampled rel err dx %.2e dw %.2e" % (edx, edw))
    assert edx <= TOL and edw <= TOL
