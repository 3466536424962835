"""GPU parity of MS-EDEN (unbiased NVFP4 backward quantization) and of the
NVFP4 linear backward built on it, against the oracle."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import msedn, nvfp4

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _check_quant(bits, axis, seed, gemm_id, stream, clip=6.0):
    x = host_f32(bits)
    src = x if axis == fq.ROW else np.ascontiguousarray(x.T)
    words = msedn.sign_mask128(seed, gemm_id)
    codes, sc, g, S = msedn.msedn_quantize(src, words, seed=seed, stream=stream, s=clip)
    out, s_gpu = fq.nv_msedn_quantize(dev_bf16(bits), axis=axis, seed=seed, gemm_id=gemm_id,
                                      stream=stream, clip=clip, want_s=True)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g, (cpu(out.tensor_scale)[0], g)
    assert_bytes_equal(cpu(s_gpu).view(np.uint32), S.view(np.uint32), "EDEN S")
    assert_bytes_equal(cpu(out.codes), codes, "ms-eden codes")
    assert_bytes_equal(cpu(out.scales), sc, "ms-eden scales")


@pytest.mark.parametrize("shape", [(32, 128), (64, 256), (96, 384), (160, 1024)])
@pytest.mark.parametrize("seed", [0, 5])
def test_msedn_row_bit_exact(shape, seed):
    log("ms-eden row", shape, seed)
    _check_quant(synth.normal_with_outliers(shape, seed, 2), fq.ROW, seed, 1, 5)


@pytest.mark.parametrize("shape", [(128, 64), (256, 96), (384, 160), (128, 32), (256, 224)])
def test_msedn_col_bit_exact(shape):
    log("ms-eden col", shape)
    _check_quant(synth.normal_with_outliers(shape, 3, 0), fq.COL, 3, 2, 8)


def test_msedn_edge_cases():
    rs = np.random.default_rng(12)
    x = (rs.standard_normal((64, 256)) * np.exp(rs.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[1] = 0.0                      # zero row
    x[2, :128] = 0.0                # zero chunk
    x[3, 5] = 1e30                  # one huge value
    x[4] = 1e-30                    # tiny row (fp32-subnormal products)
    bits = synth.f32_to_bf16_bits(x)
    _check_quant(bits, fq.ROW, 9, 1, 5)
    _check_quant(np.ascontiguousarray(np.vstack([bits, bits])[:, :96]), fq.COL, 9, 2, 7)
    # clip factor below 6 (clipping in the pseudo-scale domain)
    _check_quant(synth.normal((64, 256), 1.0, 13, 0), fq.ROW, 13, 1, 5, clip=4.0)


def test_msedn_table1_on_gpu(golden):
    """MSE of the GPU's MS-EDEN on N(0,1) matches the page's 9.8e-3."""
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    x = np.random.default_rng(0).standard_normal((1024, 1024)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    out = fq.nv_msedn_quantize(dev_bf16(bits), axis=fq.ROW, seed=0, gemm_id=1, stream=5)
    y = msedn.rht128(host_f32(bits), msedn.sign_mask128(0, 1))
    d = nvfp4.dequantize(cpu(out.codes), cpu(out.scales), cpu(out.tensor_scale)[0])
    mse = np.mean((d - y) ** 2) * 1e3
    log("  ms-eden mse x1e3", mse)
    assert abs(mse - want["ms_eden"]) < 0.3


def _oracle_bwd(dyf, xf, wf, seed):
    w1, w2 = msedn.sign_mask128(seed, 1), msedn.sign_mask128(seed, 2)
    a = msedn.msedn_quantize(dyf, w1, seed=seed, stream=5)[:3]
    b = msedn.msedn_quantize(np.ascontiguousarray(wf.T), w1, seed=seed, stream=6)[:3]
    dx = nvfp4.gemm_fp8_staged(*a, *b)
    c = msedn.msedn_quantize(np.ascontiguousarray(dyf.T), w2, seed=seed, stream=7)[:3]
    d = msedn.msedn_quantize(np.ascontiguousarray(xf.T), w2, seed=seed, stream=8)[:3]
    dw = nvfp4.gemm_fp8_staged(*c, *d)
    return dx, dw


@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 384, 160), (128, 256, 512)])
def test_nv_linear_bwd_small(m, n, k):
    log("nv bwd", m, n, k)
    xb = synth.normal((m, k), 1.0, 4, 0)
    wb = synth.normal((n, k), 0.02, 4, 1)
    dyb = synth.normal((m, n), 1e-3, 4, 2)
    dx, dw = fq.nv_linear_bwd(dev_bf16(dyb), dev_bf16(xb), dev_bf16(wb), seed=11)
    torch.cuda.synchronize()
    rdx, rdw = _oracle_bwd(host_f32(dyb), host_f32(xb), host_f32(wb), 11)
    edx, edw = rel_fro(cpu(dx), rdx), rel_fro(cpu(dw), rdw)
    log("  rel err dx %.2e dw %.2e" % (edx, edw))
    assert edx <= TOL and edw <= TOL


def test_nv_linear_bwd_unbiased_on_gpu():
    """Mean of B GPU backward estimates (different seeds) -> exact gradients."""
    m, n, k = 128, 128, 64
    xb = synth.normal((m, k), 1.0, 5, 0)
    wb = synth.normal((n, k), 1.0, 5, 1)
    dyb = synth.normal((m, n), 1.0, 5, 2)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    ex_dx = host_f32(dyb).astype(np.float64) @ host_f32(wb).astype(np.float64)
    ex_dw = host_f32(dyb).T.astype(np.float64) @ host_f32(xb).astype(np.float64)
    dxs, dws = [], []
    for seed in range(256):
        dx, dw = fq.nv_linear_bwd(dy, x, w, seed=seed)
        dxs.append(cpu(dx))
        dws.append(cpu(dw))
    for ests, ex in ((np.array(dxs), ex_dx), (np.array(dws), ex_dw)):
        def mse(B):
            mm = ests[: (len(ests) // B) * B].reshape(-1, B, *ex.shape).mean(axis=1)
            return np.mean((mm - ex) ** 2)
        e1, e16, e64 = mse(1), mse(16), mse(64)
        log("  1/B mse", e1, e16, e64)
        assert e16 < e1 / 8 and e64 < e1 / 25


@pytest.mark.timeout(600)
def test_nv_linear_bwd_full_size_sampled():
    """M=8192, N=K=4096 (the Quartet layer's dY, X, W): sampled dX / dW entries
    against oracle operands quantized row by row with the full tensors' ranges."""
    d = synth.quartet_linear(0)
    xb, wb, dyb = d["x"], d["w"], d["dy"]
    m, k = xb.shape
    n = wb.shape[0]
    seed = 0
    log("nv bwd full-size", m, n, k)
    dx, dw = fq.nv_linear_bwd(dev_bf16(dyb), dev_bf16(xb), dev_bf16(wb), seed=seed)
    torch.cuda.synchronize()
    dx, dw = cpu(dx), cpu(dw)
    xf, wf, dyf = host_f32(xb), host_f32(wb), host_f32(dyb)
    w1, w2 = msedn.sign_mask128(seed, 1), msedn.sign_mask128(seed, 2)
    rs = np.random.default_rng(321)
    ri = np.sort(rs.choice(m, 24, replace=False))
    cj = np.sort(rs.choice(n, 24, replace=False))
    ck = np.sort(rs.choice(k, 24, replace=False))
    wt, dyt, xt = np.ascontiguousarray(wf.T), np.ascontiguousarray(dyf.T), np.ascontiguousarray(xf.T)
    # global range exponents of the four operands (whole tensors), then rows
    k_a = msedn.msedn_range_exponent(dyf, w1)
    k_b = msedn.msedn_range_exponent(wt, w1)
    a = msedn.msedn_quantize(dyf[ri], w1, seed=seed, stream=5, row_ids=ri, k=k_a)[:3]
    b = msedn.msedn_quantize(wt[ck], w1, seed=seed, stream=6, row_ids=ck, k=k_b)[:3]
    edx = rel_fro(dx[np.ix_(ri, ck)], nvfp4.gemm_fp8_staged(*a, *b))
    k_c = msedn.msedn_range_exponent(dyt, w2)
    k_d = msedn.msedn_range_exponent(xt, w2)
    c = msedn.msedn_quantize(dyt[cj], w2, seed=seed, stream=7, row_ids=cj, k=k_c)[:3]
    dd = msedn.msedn_quantize(xt[ck], w2, seed=seed, stream=8, row_ids=ck, k=k_d)[:3]
    edw = rel_fro(dw[np.ix_(cj, ck)], nvfp4.gemm_fp8_staged(*c, *dd))
    log("  sampled rel err dx %.2e dw %.2e" % (edx, edw))
    assert edx <= TOL and edw <= TOL


def _check_sr(bits, seed, stream):
    codes, sc, g = msedn.sr_quantize(host_f32(bits), seed=seed, stream=stream)
    out = fq.nv_sr_quantize(dev_bf16(bits), seed=seed, stream=stream)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g, (cpu(out.tensor_scale)[0], g)
    assert_bytes_equal(cpu(out.scales), sc, "sr scales")
    assert_bytes_equal(cpu(out.codes), codes, "sr codes")


@pytest.mark.parametrize("shape", [(32, 32), (64, 256), (96, 1056), (352, 160)])
@pytest.mark.parametrize("seed", [0, 21])
def test_nv_sr_bit_exact(shape, seed):
    log("nvfp4 sr", shape, seed)
    _check_sr(synth.normal_with_outliers(shape, seed, 1), seed, 3)


def test_nv_sr_edge_cases():
    rs = np.random.default_rng(4)
    x = (rs.standard_normal((32, 64)) * np.exp(rs.uniform(-30, 30, (32, 1)))).astype(np.float32)
    x[1] = 0.0
    x[2, :16] = -0.0
    x[3, 7] = 3e38
    x[5] = 1e-38
    _check_sr(synth.f32_to_bf16_bits(x), 2, 1)
    _check_sr(synth.f32_to_bf16_bits(np.zeros((32, 32), np.float32)), 2, 1)
    # groups with normal scales holding: -0 beside nonzero values (the
    # quotient keeps x's sign); bf16 subnormals and tiny quotients (below
    # 2^-23, rounded to a signed zero) beside normal values; one repeated
    # value (every element at the group maximum)
    y = rs.standard_normal((32, 64)).astype(np.float32)
    y[6, :16] = np.where(np.arange(16) % 2 == 0, -0.0, rs.standard_normal(16))
    y[8, 16:32] = np.concatenate([[1.0, -2.0, 1e-39, -1e-39, 5e-40, -5e-40],
                                  np.ldexp(rs.choice([-1.0, 1.0], 10), -rs.integers(20, 60, 10))])
    y[10, :16] = 3.25
    y[10, 16:32] = -3.25
    _check_sr(synth.f32_to_bf16_bits(y), 5, 3)


@pytest.mark.parametrize("scale", [1e-38, 1e-30, 1e-12, 1.0, 1e12, 1e36])
def test_nv_sr_scale_range(scale):
    """Tensors across the fp32 range: the per-element quotient x / d is taken
    by Markstein's correction only for 2^-75 <= d <= 2^100 and quotients of at
    least 2^-25, and by exact division otherwise (tiny and huge tensors, tiny
    elements beside normal ones); codes and scales stay bit-exact."""
    log("nvfp4 sr scale", scale)
    rs = np.random.default_rng(12)
    x = (rs.standard_normal((64, 256)) * scale).astype(np.float32)
    x[7, :5] *= np.float32(1e-9)
    x[9, 16:32] = 0.0
    _check_sr(synth.f32_to_bf16_bits(x), 3, 2)


@pytest.mark.parametrize("scale", [1e-38, 1e-30, 1e12, 1e30])
def test_msedn_scale_range(scale):
    """MS-EDEN across the fp32 range (the pseudo-scale reciprocal is the
    hardware one only for pseudo-scales in [2^-126, 2^126])."""
    log("msedn scale", scale)
    rs = np.random.default_rng(13)
    x = (rs.standard_normal((128, 256)) * scale).astype(np.float32)
    x[7, :5] *= np.float32(1e-9)
    bits = synth.f32_to_bf16_bits(x)
    _check_quant(bits, fq.ROW, 5, 1, 5)
    _check_quant(bits, fq.COL, 5, 2, 7)


def test_nv_sr_table1_on_gpu(golden):
    """MSE of the GPU's standard NVFP4 SR on N(0,1) matches the page's 23.5e-3."""
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    x = np.random.default_rng(0).standard_normal((1024, 1024)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    out = fq.nv_sr_quantize(dev_bf16(bits), seed=0, stream=5)
    d = nvfp4.dequantize(cpu(out.codes), cpu(out.scales), cpu(out.tensor_scale)[0])
    mse = np.mean((d - host_f32(bits)) ** 2) * 1e3
    log("  sr mse x1e3", mse)
    assert abs(mse - want["sr"]) < 0.3


@pytest.mark.timeout(300)
def test_nv_sr_full_size_sampled():
    """dY of the Quartet layer (8192 x 4096): the first 1024 rows against the
    oracle run on those rows plus one appended row that carries the whole
    tensor's max (so g, and every RNG index row * cols + col, are the same)."""
    dyb = synth.quartet_linear(0)["dy"]
    out = fq.nv_sr_quantize(dev_bf16(dyb), seed=7, stream=2)
    torch.cuda.synchronize()
    dyf = host_f32(dyb)
    amax = np.max(np.abs(dyf))
    sub = np.vstack([dyf[:1024], np.full((1, dyf.shape[1]), amax, np.float32)])
    codes, sc, g = msedn.sr_quantize(sub, seed=7, stream=2)
    log("nvfp4 sr full-size", dyf.shape)
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.codes)[:1024], codes[:1024], "sr codes, first 1024 rows")
    assert_bytes_equal(cpu(out.scales)[:1024], sc[:1024], "sr scales, first 1024 rows")
