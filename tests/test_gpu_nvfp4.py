"""GPU parity of the NVFP4 forward variant (RTN + Four-over-Six, FP8-staged GEMM)."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import nvfp4

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.mark.parametrize("shape", [(64, 128), (96, 160), (32, 32), (512, 1024)])
@pytest.mark.parametrize("use46", [True, False])
def test_quantize46_bit_exact(shape, use46):
    log("nv quant", shape, use46)
    bits = synth.normal_with_outliers(shape, 5, 0)
    out = fq.nv_quantize46(dev_bf16(bits), use46)
    torch.cuda.synchronize()
    c, s, g = nvfp4.quantize46(host_f32(bits), use46)
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.scales), s, "nv scales")
    assert_bytes_equal(cpu(out.codes), c, "nv codes")


def test_quantize46_wide_range_blocks():
    rs = np.random.default_rng(7)
    x = (rs.standard_normal((64, 256)) * np.exp(rs.uniform(-12, 8, (64, 1)))).astype(np.float32)
    x[3, :16] = 0.0
    x[5, 16:32] = 1e-30
    bits = synth.f32_to_bf16_bits(x)
    out = fq.nv_quantize46(dev_bf16(bits), True)
    torch.cuda.synchronize()
    c, s, g = nvfp4.quantize46(host_f32(bits), True)
    assert_bytes_equal(cpu(out.scales), s, "nv scales")
    assert_bytes_equal(cpu(out.codes), c, "nv codes")


def test_table1_mse_from_gpu_codes(golden):
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    x = np.random.default_rng(0).standard_normal((1024, 1024)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    xf = host_f32(bits)
    for name, use46 in (("rtn", False), ("rtn_46", True)):
        out = fq.nv_quantize46(dev_bf16(bits), use46)
        d = nvfp4.dequantize(cpu(out.codes), cpu(out.scales), cpu(out.tensor_scale)[0])
        mse = np.mean((d - xf) ** 2) * 1e3
        log("  table1", name, mse, "printed", want[name])
        assert abs(mse - want[name]) < 0.3


def _nv_dev(q):
    c, s, g = q
    return fq.NVTensor(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                       torch.tensor([g], dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("m,n,k", [(64, 64, 128), (96, 160, 320), (256, 256, 1024), (32, 64, 32)])
def test_nv_gemm_parity(m, n, k):
    log("nv gemm", m, n, k)
    a = nvfp4.quantize46(host_f32(synth.normal((m, k), 1.0, 6, 0)))
    b = nvfp4.quantize46(host_f32(synth.normal((n, k), 0.02, 6, 1)))
    c = cpu(fq.nv_gemm(_nv_dev(a), _nv_dev(b)))
    want = nvfp4.gemm_fp8_staged(*a, *b)
    err = rel_fro(c, want)
    exact = rel_fro(c, nvfp4.gemm_exact(*a, *b))
    log("  rel err vs staged %.2e, vs exact NVFP4 product %.2e" % (err, exact))
    assert err <= TOL


def test_nv_linear_tiny():
    xb = synth.normal((64, 128), 1.0, 8, 0)
    wb = synth.normal((96, 128), 0.02, 8, 1)
    y = cpu(fq.nv_linear_fwd(dev_bf16(xb), dev_bf16(wb)))
    want, _, _ = nvfp4.linear_fwd(host_f32(xb), host_f32(wb))
    assert rel_fro(y, want) <= TOL


def test_nvfp4_workload_full_size_sampled():
    """16384 x 8192 -> 8192, X ~ N(0,1), W ~ N(0,0.02): sampled outputs."""
    d = synth.nvfp4_linear(0)
    xb, wb = d["x"], d["w"]
    m, k = xb.shape
    n = wb.shape[0]
    log("nv full-size", m, n, k)
    y = cpu(fq.nv_linear_fwd(dev_bf16(xb), dev_bf16(wb)))
    xf, wf = host_f32(xb), host_f32(wb)
    gx = nvfp4.tensor_scale(xf)
    gw = nvfp4.tensor_scale(wf)
    rs = np.random.default_rng(9)
    ri = np.sort(rs.choice(m, 48, replace=False))
    cj = np.sort(rs.choice(n, 48, replace=False))
    qx = nvfp4.quantize46(xf[ri], True, g=gx)
    qw = nvfp4.quantize46(wf[cj], True, g=gw)
    err = rel_fro(y[np.ix_(ri, cj)], nvfp4.gemm_fp8_staged(*qx, *qw))
    log("  sampled rel err %.2e" % err)
    assert err <= TOL
