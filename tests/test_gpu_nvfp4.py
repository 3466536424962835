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


@pytest.mark.parametrize("shape", [(32, 96), (1056, 4128), (4160, 8192)])
def test_tensor_scale_max_position(shape):
    """g = fl32(max|x| / 1536) with the largest magnitude planted first, last
    and in the middle of the tensor, negative or positive.  The chunk counts
    (16 B each) are not multiples of a workgroup's 2048, and the largest shape
    (4.26 M chunks) takes two passes of the flat reduction's grid."""
    r, c = shape
    base = synth.normal(shape, 1.0, 11, 0)
    for pos, val in ((0, -50.0), (r * c - 1, 60.0), (r * c // 2 + 7, -70.0)):
        bits = base.copy().reshape(-1)
        bits[pos] = synth.f32_to_bf16_bits(np.array([val], dtype=np.float32))[0]
        bits = bits.reshape(shape)
        log("tensor scale", shape, "max at", pos)
        out = fq.nv_quantize46(dev_bf16(bits), True)
        torch.cuda.synchronize()
        g = nvfp4.tensor_scale(host_f32(bits))
        assert cpu(out.tensor_scale)[0] == g


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


def test_quantize46_signed_zeros_and_subnormals():
    """Groups with normal scales holding -0 beside nonzero values (the code
    keeps x's sign bit), bf16 subnormals and tiny values beside normal ones,
    and one repeated value."""
    rs = np.random.default_rng(8)
    x = rs.standard_normal((32, 64)).astype(np.float32)
    x[2, :16] = np.where(np.arange(16) % 2 == 0, -0.0, rs.standard_normal(16))
    x[3, 16:32] = np.where(np.arange(16) % 3 == 0, 0.0, -rs.random(16))
    x[4, :16] = np.concatenate([[1.0, -2.0, 1e-39, -1e-39, 5e-40, -5e-40],
                                np.ldexp(rs.choice([-1.0, 1.0], 10), -rs.integers(20, 60, 10))])
    x[5, :16] = -2.5
    bits = synth.f32_to_bf16_bits(x)
    for use46 in (True, False):
        out = fq.nv_quantize46(dev_bf16(bits), use46)
        torch.cuda.synchronize()
        c, s, g = nvfp4.quantize46(host_f32(bits), use46)
        assert_bytes_equal(cpu(out.scales), s, "nv scales")
        assert_bytes_equal(cpu(out.codes), c, "nv codes")


@pytest.mark.parametrize("scale", [1e-38, 1e-30, 1e-12, 1.0, 1e12, 1e36])
def test_quantize46_scale_range(scale):
    """Tensors across the fp32 range.  The quotients amax_b / (c g) and
    x / d take shortcuts (Markstein's correction, the hardware reciprocal
    inside a bracket) only where their arguments are in range, and divide
    exactly elsewhere; codes and scales stay bit-exact throughout."""
    log("nv quant scale", scale)
    rs = np.random.default_rng(11)
    x = (rs.standard_normal((64, 256)) * scale).astype(np.float32)
    x[7, :5] *= np.float32(1e-9)          # tiny elements beside normal ones
    x[9, 16:32] = 0.0
    bits = synth.f32_to_bf16_bits(x)
    for use46 in (True, False):
        out = fq.nv_quantize46(dev_bf16(bits), use46)
        torch.cuda.synchronize()
        c, s, g = nvfp4.quantize46(host_f32(bits), use46)
        assert cpu(out.tensor_scale)[0] == g
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


def _random_nv_operand(rows, cols, seed, zero_blocks=True):
    """Random E2M1 code bytes and positive E4M3 scale bytes (normal and
    subnormal, some zero; with zero_blocks, some 32-blocks with both scales 0)."""
    rs = np.random.default_rng(seed)
    codes = rs.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rs.integers(0, 0x7F, (rows, cols // 16), dtype=np.uint8)     # 0x7F is NaN
    scales[rs.random(scales.shape) < 0.05] = 0
    scales[rs.random(scales.shape) < 0.1] &= 0x07                          # subnormal scales
    if zero_blocks:
        zb = rs.random((rows, cols // 32)) < 0.03
        scales.reshape(rows, cols // 32, 2)[zb] = 0
    return codes, scales


def _staged_from_workspace(m, n, k, a, b, row_sample=None):
    """Run fp4nv_gemm through the C ABI and read the FP8-staged operands back
    from its workspace (A's E4M3 [m, k] and E8M0 [m, k/32], then B's, each
    piece 256-B aligned)."""
    from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
    L = fq.lib()
    ru = lambda v: (v + 255) // 256 * 256
    ws = torch.empty(L.fp4nv_gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    dev = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()
    ac, asc, bc, bsc = dev(a[0]), dev(a[1]), dev(b[0]), dev(b[1])
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    _check(L.fp4nv_gemm(_ptr(ac), _ptr(asc), _ptr(one), _ptr(bc), _ptr(bsc), _ptr(one), m, n, k,
                        _ptr(c), n, _ptr(ws), ws.numel(), _stream()))
    torch.cuda.synchronize()
    o = 0
    fa = ws[o:o + m * k].view(m, k); o += ru(m * k)
    ea = ws[o:o + m * k // 32].view(m, k // 32); o += ru(m * k // 32)
    fb = ws[o:o + n * k].view(n, k); o += ru(n * k)
    eb = ws[o:o + n * k // 32].view(n, k // 32)
    if row_sample is not None:
        ra, rb = row_sample
        return cpu(fa[ra]), cpu(ea[ra]), cpu(fb[rb]), cpu(eb[rb])
    return cpu(fa), cpu(ea), cpu(fb), cpu(eb)


@pytest.mark.parametrize("m,n,k", [(64, 32, 128), (96, 160, 320), (256, 64, 1024), (32, 32, 32)])
def test_fp8_staging_bytes_exact(m, n, k):
    """The staged E4M3 bytes and E8M0 block scales equal the oracle's staging
    bit for bit (byte work), including zero and subnormal E4M3 scales, blocks
    whose two scales are both 0, and negative zero codes."""
    log("fp8 staging", m, n, k)
    a, b = _random_nv_operand(m, k, 21), _random_nv_operand(n, k, 22)
    fa, ea, fb, eb = _staged_from_workspace(m, n, k, a, b)
    for what, got_f, got_e, op in (("A", fa, ea, a), ("B", fb, eb, b)):
        want_f, want_e = nvfp4.fp8_stage_bytes(*op)
        assert_bytes_equal(got_f, want_f, what + " staged E4M3")
        assert_bytes_equal(got_e, (want_e + 127).astype(np.uint8), what + " E8M0 block scales")


def test_fp8_staging_bytes_full_size_sampled():
    """NVFP4 workload shape (M=16384, N=K=8192) in the forward's launch
    configuration; staging is row-independent, so sampled rows of both staged
    operands are compared with the oracle bit for bit."""
    m, n, k = 16384, 8192, 8192
    log("fp8 staging full size", m, n, k)
    a, b = _random_nv_operand(m, k, 23), _random_nv_operand(n, k, 24)
    rs = np.random.default_rng(25)
    ra = np.sort(np.concatenate([[0, m - 1], rs.choice(m, 30, replace=False)]))
    rb = np.sort(np.concatenate([[0, n - 1], rs.choice(n, 30, replace=False)]))
    fa, ea, fb, eb = _staged_from_workspace(m, n, k, a, b, (torch.from_numpy(ra).cuda(),
                                                             torch.from_numpy(rb).cuda()))
    for what, got_f, got_e, op, rows in (("A", fa, ea, a, ra), ("B", fb, eb, b, rb)):
        want_f, want_e = nvfp4.fp8_stage_bytes(op[0][rows], op[1][rows])
        assert_bytes_equal(got_f, want_f, what + " staged E4M3 (sampled rows)")
        assert_bytes_equal(got_e, (want_e + 127).astype(np.uint8), what + " E8M0 (sampled rows)")
