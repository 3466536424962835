"""Every bf16-input entry point on rows padded beyond `cols` (leading dimension
ld > cols): the padding is never read and the results equal the oracle's on
the unpadded matrix, bit for bit."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import msedn, mx, nvfp4, quest, rng

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log

pytestmark = pytest.mark.gpu

ROWS, COLS, LD = 256, 384, 448


def _padded(seed):
    """bf16 bits [ROWS, LD] whose padding holds NaNs, and the device view [ROWS, COLS]."""
    bits = synth.normal_with_outliers((ROWS, LD), seed, 0)
    bits[:, COLS:] = 0x7FC0                       # NaN: would poison any group that read it
    return bits, dev_bf16(bits)[:, :COLS]


def test_mx_col_and_dual_strided():
    bits, x = _padded(1)
    xf = host_f32(bits)[:, :COLS]
    m1, m2 = rng.sign_mask(4, 1), rng.sign_mask(4, 2)
    log("strided mx col / dual")
    out = fq.hadamard_quantize(x, axis=fq.COL, rounding=fq.SR, mask=m2, seed=4, rng_stream=3)
    want = mx.quantize(xf, rounding=mx.SR, axis=mx.COL, sign_mask=m2, seed=4, stream=3)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(out.codes), want[0], "col codes")
    assert_bytes_equal(cpu(out.scales), want[1], "col scales")
    ro, co = fq.hadamard_quantize_dual(x, fq.RTN, m1, 0, fq.SR, m2, 4, seed=4)
    wr = mx.quantize(xf, rounding=mx.RTN, axis=mx.ROW, sign_mask=m1)
    wc = mx.quantize(xf, rounding=mx.SR, axis=mx.COL, sign_mask=m2, seed=4, stream=4)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(ro.codes), wr[0], "dual row codes")
    assert_bytes_equal(cpu(co.codes), wc[0], "dual col codes")
    assert_bytes_equal(cpu(co.scales), wc[1], "dual col scales")


def test_quest_strided():
    bits, x = _padded(2)
    m = rng.sign_mask(5, 0)
    log("strided quest")
    out, mk = fq.quest_quantize(x, mask=m)
    codes, sc, wm = quest.quest_quantize(host_f32(bits)[:, :COLS], m, fq.QUEST_CLIP)
    torch.cuda.synchronize()
    assert_bytes_equal(cpu(out.codes), codes, "quest codes")
    assert_bytes_equal(cpu(out.scales), sc, "quest scales")
    assert_bytes_equal(cpu(mk), wm, "quest mask")


def test_nvfp4_strided():
    bits, x = _padded(3)
    xf = host_f32(bits)[:, :COLS]
    log("strided nvfp4 4/6 and SR")
    out = fq.nv_quantize46(x)
    codes, sc, g = nvfp4.quantize46(xf, True)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.codes), codes, "4/6 codes")
    assert_bytes_equal(cpu(out.scales), sc, "4/6 scales")
    out = fq.nv_sr_quantize(x, seed=6, stream=2)
    codes, sc, g = msedn.sr_quantize(xf, seed=6, stream=2)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.codes), codes, "sr codes")
    assert_bytes_equal(cpu(out.scales), sc, "sr scales")


@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
def test_msedn_strided(axis):
    bits, x = _padded(4)
    xf = host_f32(bits)[:, :COLS]
    src = xf if axis == fq.ROW else np.ascontiguousarray(xf.T)
    log("strided ms-eden", axis)
    words = msedn.sign_mask128(7, 1)
    codes, sc, g, _ = msedn.msedn_quantize(src, words, seed=7, stream=5)
    out = fq.nv_msedn_quantize(x, axis=axis, seed=7, gemm_id=1, stream=5)
    torch.cuda.synchronize()
    assert cpu(out.tensor_scale)[0] == g
    assert_bytes_equal(cpu(out.codes), codes, "ms-eden codes")
    assert_bytes_equal(cpu(out.scales), sc, "ms-eden scales")
