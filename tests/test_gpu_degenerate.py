"""GPU parity on whole tensors of zeros, the degenerate case where every
tensor-wide maximum is 0 (NVFP4 tensor scale, MS-EDEN range alignment) and
every group of every family is empty: codes, scales and tensor scales equal
the oracle's bit for bit, and the linear layers return exact zeros (no NaN)."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from oracle import msedn, mx, nvfp4, quest, rng

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log

pytestmark = pytest.mark.gpu

R, C = 128, 256


@pytest.fixture(scope="module")
def zeros():
    bits = np.zeros((R, C), dtype=np.uint16)
    return bits, dev_bf16(bits), host_f32(bits)


def test_zero_tensor_mx_and_quest(zeros):
    _, x, xf = zeros
    m = rng.sign_mask(3, 0)
    log("zeros: mx, quest")
    for axis in (fq.ROW, fq.COL):
        for rnd in (fq.RTN, fq.SR):
            out = fq.hadamard_quantize(x, axis=axis, rounding=rnd, mask=m, seed=2, rng_stream=1)
            wc, ws = mx.quantize(xf, rounding=rnd, axis=axis, sign_mask=m, seed=2, stream=1)
            torch.cuda.synchronize()
            assert_bytes_equal(cpu(out.codes), wc, "mx codes")
            assert_bytes_equal(cpu(out.scales), ws, "mx scales")
    qo, qm = fq.quest_quantize(x, mask=m)
    wc, ws, wm = quest.quest_quantize(xf, m, fq.QUEST_CLIP)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(qo.codes), wc, "quest codes")
    assert_bytes_equal(cpu(qo.scales), ws, "quest scales")
    assert_bytes_equal(cpu(qm), wm, "quest mask")


@pytest.mark.parametrize("use46", [True, False])
def test_zero_tensor_nvfp4(zeros, use46):
    _, x, xf = zeros
    log("zeros: nvfp4 4/6", use46)
    out = fq.nv_quantize46(x, use46)
    c, s, g = nvfp4.quantize46(xf, use46)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.codes), c, "nv codes")
    assert_bytes_equal(cpu(out.scales), s, "nv scales")


@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
def test_zero_tensor_msedn(zeros, axis):
    _, x, xf = zeros
    log("zeros: ms-eden", axis)
    src = xf if axis == fq.ROW else np.ascontiguousarray(xf.T)
    codes, sc, g, S = msedn.msedn_quantize(src, msedn.sign_mask128(4, 1), seed=4, stream=5)
    out, s_gpu = fq.nv_msedn_quantize(x, axis=axis, seed=4, gemm_id=1, stream=5, want_s=True)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(s_gpu).view(np.uint32), S.view(np.uint32), "EDEN S")
    assert_bytes_equal(cpu(out.codes), codes, "ms-eden codes")
    assert_bytes_equal(cpu(out.scales), sc, "ms-eden scales")


def test_zero_tensor_linear_layers(zeros):
    _, x, _ = zeros
    w = x[:128].contiguous()                  # NVFP4 backward wants m, n multiples of 128
    dy = torch.zeros((R, 128), dtype=torch.bfloat16, device="cuda")
    log("zeros: linear layers")
    y, ctx = fq.linear_fwd(x, w, seed=1)
    dx, dw = fq.linear_bwd(dy, ctx)
    ny = fq.nv_linear_fwd(x, w)
    ndx, ndw = fq.nv_linear_bwd(dy, x, w, seed=1)
    torch.cuda.synchronize()
    for name, t in (("y", y), ("dx", dx), ("dw", dw), ("nv y", ny), ("nv dx", ndx), ("nv dw", ndw)):
        a = cpu(t)
        assert np.all(a == 0.0), name
