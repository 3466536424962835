"""GPU parity: the MXFP4 GEMM against the oracle's float64 dequantized product."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import mx

from gpu_util import assert_gemm_close, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-5   # relative Frobenius error against the fp64 product


def _operands(m, n, k, seed=0):
    a = synth.normal_with_outliers((m, k), seed, 0)
    b = synth.normal((n, k), 0.02, seed, 1)
    return a, b


def _to_dev_mx(codes, scales):
    return fq.MXTensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())


@pytest.mark.parametrize("m,n,k", [(64, 128, 128), (32, 32, 32), (96, 160, 320), (128, 128, 256),
                                   (256, 384, 1024), (160, 96, 288), (512, 256, 2048),
                                   (288, 224, 384), (544, 480, 1152), (768, 512, 640),
                                   (544, 480, 2048), (96, 800, 3072)])
def test_gemm_parity(m, n, k):
    log("gemm", m, n, k)
    a, b = _operands(m, n, k)
    qa = mx.quantize(host_f32(a), rounding=mx.RTN, sign_mask=3)
    qb = mx.quantize(host_f32(b), rounding=mx.SR, sign_mask=3, seed=1, stream=2)
    c = fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb), alpha=1.5)
    torch.cuda.synchronize()
    assert_gemm_close(cpu(c), mx.dequantize(*qa), mx.dequantize(*qb), 1.5, "gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(512, 1024, 512), (1024, 2048, 256), (1056, 1824, 320),
                                   (2048, 1024, 1024)])
def test_gemm_parity_xcd_remap(m, n, k):
    """Shapes whose 256 x 256 tile count is a multiple of 8 (8, 32, 40 and 32
    tiles), so the launch takes the XCD-aware tile order; one is ragged in M,
    N and K.  C starts as NaN: an unwritten or twice-mapped tile fails."""
    log("gemm remap", m, n, k, "tiles", -(-m // 256) * -(-n // 256))
    a, b = _operands(m, n, k, seed=2)
    qa = mx.quantize(host_f32(a), rounding=mx.SR, sign_mask=7, seed=5, stream=1)
    qb = mx.quantize(host_f32(b), rounding=mx.RTN, sign_mask=7)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb), alpha=16 / 9, out=out)
    torch.cuda.synchronize()
    c = cpu(out)
    assert np.all(np.isfinite(c))
    assert_gemm_close(c, mx.dequantize(*qa), mx.dequantize(*qb), mx.ALPHA_BWD, "remap %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k,off", [(256, 512, 1024, 1), (288, 544, 4096, 8), (512, 256, 2560, 4)])
def test_gemm_scale_pointer_alignment(m, n, k, off):
    """Scale pointers off 16-B alignment (byte offsets 1, 8, 4) take the
    per-stage scale loads; aligned ones with K/32 a multiple of 16 take the
    16-B loads every second stage.  Both are bit-identical and match the
    oracle's product element-wise."""
    log("gemm scale alignment", m, n, k, off)
    a, b = _operands(m, n, k, seed=4)
    qa = mx.quantize(host_f32(a), rounding=mx.SR, sign_mask=5, seed=2, stream=3)
    qb = mx.quantize(host_f32(b), rounding=mx.RTN, sign_mask=5)

    def shifted(scales):
        buf = torch.zeros(scales.size + 32, dtype=torch.uint8, device="cuda")
        t = buf[off:off + scales.size].view(scales.shape)
        t.copy_(torch.from_numpy(scales))
        assert t.data_ptr() % 16 == off % 16
        return t

    c0 = fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb), alpha=1.25)
    c1 = fq.gemm(fq.MXTensor(torch.from_numpy(qa[0]).cuda(), shifted(qa[1])),
                 fq.MXTensor(torch.from_numpy(qb[0]).cuda(), shifted(qb[1])), alpha=1.25)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    assert_gemm_close(cpu(c1), mx.dequantize(*qa), mx.dequantize(*qb), 1.25, "scale alignment")


def test_gemm_output_stride_and_alpha():
    a, b = _operands(64, 96, 256)
    qa = mx.quantize(host_f32(a), rounding=mx.RTN)
    qb = mx.quantize(host_f32(b), rounding=mx.RTN)
    out = torch.full((64, 128), 7.0, dtype=torch.float32, device="cuda")
    fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb), alpha=16 / 9, out=out)
    torch.cuda.synchronize()
    o = cpu(out)
    assert np.all(o[:, 96:] == 7.0)               # columns beyond n untouched
    assert_gemm_close(o[:, :96], mx.dequantize(*qa), mx.dequantize(*qb), 16 / 9, "strided out")


def test_gemm_nan_scale_propagates():
    a, b = _operands(64, 64, 128)
    qa = list(mx.quantize(host_f32(a), rounding=mx.RTN))
    qb = mx.quantize(host_f32(b), rounding=mx.RTN)
    qa[1] = qa[1].copy()
    qa[1][3, 1] = 255                              # non-finite group in row 3
    c = cpu(fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb)))
    assert np.all(np.isnan(c[3]))
    assert np.all(np.isfinite(np.delete(c, 3, axis=0)))


def test_gemm_extreme_scales():
    # products spanning the E8M0 range stay exact in fp32 accumulation
    rs = np.random.default_rng(0)
    qa = (rs.integers(0, 256, (64, 64), dtype=np.uint8), rs.integers(100, 150, (64, 4)).astype(np.uint8))
    qb = (rs.integers(0, 256, (32, 64), dtype=np.uint8), rs.integers(100, 150, (32, 4)).astype(np.uint8))
    c = cpu(fq.gemm(_to_dev_mx(*qa), _to_dev_mx(*qb)))
    assert_gemm_close(c, mx.dequantize(*qa), mx.dequantize(*qb), 1.0, "extreme scales")


def _bf16_rne_bits(f32):
    """fp32 -> bf16 bits, round to nearest even (the input generators' rounding)."""
    return synth.f32_to_bf16_bits(np.asarray(f32, dtype=np.float32))


@pytest.mark.parametrize("m,n,k,ldc", [(256, 256, 256, 256), (352, 160, 96, 168), (96, 544, 320, 552),
                                       (32, 32, 32, 40)])
def test_gemm_bf16_output(m, n, k, ldc):
    """The bf16-output GEMM writes exactly bf16_RNE of the fp32 GEMM's value, and
    agrees with the oracle's fp64 product rounded to bf16 (up to the fp32
    accumulation crossing a rounding boundary: rare, and then one bf16 ulp)."""
    log("gemm bf16 out", m, n, k, ldc)
    a, b = _operands(m, n, k, seed=4)
    qa = mx.quantize(host_f32(a), rounding=mx.SR, sign_mask=5, seed=3, stream=1)
    qb = mx.quantize(host_f32(b), rounding=mx.SR, sign_mask=5, seed=3, stream=2)
    A, B = _to_dev_mx(*qa), _to_dev_mx(*qb)
    c32 = fq.gemm(A, B, alpha=16 / 9)
    c16 = torch.full((m, ldc), 3.0, dtype=torch.bfloat16, device="cuda")
    fq.gemm_bf16(A, B, alpha=16 / 9, out=c16[:, :n])
    torch.cuda.synchronize()
    got = cpu(c16.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got[:, :n], _bf16_rne_bits(cpu(c32)))
    assert np.all(got[:, n:] == 0x4040)                   # padding (3.0) untouched
    want = _bf16_rne_bits(mx.gemm(*qa, *qb, alpha=mx.ALPHA_BWD).astype(np.float32))
    diff = np.abs(got[:, :n].astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and np.mean(diff > 0) < 1e-3


def test_gemm_bf16_output_full_size():
    """Quartet workload shape (8192 x 4096, K 4096), launch as the step uses it:
    the bf16 output equals bf16_RNE of the fp32 GEMM bit for bit."""
    m, n, k = 8192, 4096, 4096
    log("gemm bf16 out full size", m, n, k)
    g = torch.Generator(device="cuda").manual_seed(11)
    A = fq.MXTensor(torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device="cuda", generator=g),
                    torch.randint(118, 130, (m, k // 32), dtype=torch.uint8, device="cuda", generator=g))
    B = fq.MXTensor(torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device="cuda", generator=g),
                    torch.randint(118, 130, (n, k // 32), dtype=torch.uint8, device="cuda", generator=g))
    c32 = fq.gemm(A, B)
    c16 = fq.gemm_bf16(A, B)
    torch.cuda.synchronize()
    assert np.array_equal(cpu(c16.view(torch.int16)).view(np.uint16), _bf16_rne_bits(cpu(c32)))
