"""GPU parity: the HIP RHT + MXFP4 quantizers against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import mx, rng

from gpu_util import assert_bytes_equal, cpu, dev_bf16, edge_case_tensor, edge_case_tensor_cols, host_f32, log

pytestmark = pytest.mark.gpu

SHAPES = [(64, 128), (96, 160), (32, 32), (256, 1024), (160, 96)]


def _oracle(xf, axis, rounding, had, mask, seed, stream):
    return mx.quantize(xf, rounding=rounding, axis=axis, hadamard=had, sign_mask=mask, seed=seed,
                       stream=stream)


def _check(bits, axis, rounding, had, mask=0x9E3779B9, seed=5, stream=3, what=""):
    log("quant", what, bits.shape, "axis", axis, "round", rounding, "had", had)
    out = fq.quantize(dev_bf16(bits), axis=axis, rounding=rounding, seed=seed, rng_stream=stream,
                      hadamard=had, mask=mask)
    torch.cuda.synchronize()
    want_c, want_s = _oracle(host_f32(bits), axis, rounding, had, mask, seed, stream)
    assert_bytes_equal(cpu(out.scales), want_s, what + " scales")
    assert_bytes_equal(cpu(out.codes), want_c, what + " codes")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
@pytest.mark.parametrize("rounding", [fq.RTN, fq.SR])
@pytest.mark.parametrize("had", [True, False])
def test_quantize_small(shape, axis, rounding, had):
    bits = synth.normal_with_outliers(shape, seed=1, tensor_id=0)
    _check(bits, axis, rounding, had, what="small")


@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
@pytest.mark.parametrize("rounding", [fq.RTN, fq.SR])
@pytest.mark.parametrize("had", [True, False])
def test_quantize_edge_cases(axis, rounding, had):
    bits = edge_case_tensor(128, 256)
    _check(bits, axis, rounding, had, what="edge")


@pytest.mark.parametrize("rounding", [fq.RTN, fq.SR])
@pytest.mark.parametrize("had", [True, False])
@pytest.mark.parametrize("shape", [(256, 128), (160, 96)])
def test_quantize_edge_cases_along_columns(rounding, had, shape):
    """The special groups planted down columns, so the column-axis quantizer
    meets whole zero, -0, subnormal, huge, tie, NaN and Inf groups."""
    bits = edge_case_tensor_cols(*shape, seed=2)
    _check(bits, fq.COL, rounding, had, what="edge-col")


@pytest.mark.parametrize("rr,cr", [(fq.RTN, fq.SR), (fq.SR, fq.SR), (fq.RTN, fq.RTN), (fq.SR, fq.RTN)])
@pytest.mark.parametrize("planted", ["rows", "cols"])
def test_dual_edge_cases(rr, cr, planted):
    """Dual kernel on tensors whose special groups run along rows or along
    columns: both outputs equal the oracle's single-axis quantizers."""
    bits = edge_case_tensor(256, 192, 6) if planted == "rows" else edge_case_tensor_cols(256, 192, 6)
    seed, m1, m2 = 3, 0x0F0F1234, 0xA5A5A5A5
    log("dual edge", planted, rr, cr)
    ro, co = fq.hadamard_quantize_dual(dev_bf16(bits), rr, m1, 1, cr, m2, 3, seed=seed)
    torch.cuda.synchronize()
    xf = host_f32(bits)
    wr = _oracle(xf, mx.ROW, rr, True, m1, seed, 1)
    wc = _oracle(xf, mx.COL, cr, True, m2, seed, 3)
    assert_bytes_equal(cpu(ro.codes), wr[0], "dual row codes")
    assert_bytes_equal(cpu(ro.scales), wr[1], "dual row scales")
    assert_bytes_equal(cpu(co.codes), wc[0], "dual col codes")
    assert_bytes_equal(cpu(co.scales), wc[1], "dual col scales")


def test_quantize_mask_zero_is_plain_hadamard():
    bits = synth.normal((64, 256), 1.0, seed=2, tensor_id=0)
    _check(bits, fq.ROW, fq.RTN, True, mask=0, what="mask0")


@pytest.mark.parametrize("rr,cr", [(fq.RTN, fq.SR), (fq.SR, fq.SR), (fq.RTN, fq.RTN)])
@pytest.mark.parametrize("shape", [(128, 64), (96, 160), (384, 320)])
def test_dual_matches_two_single_quantizers(rr, cr, shape):
    bits = synth.normal_with_outliers(shape, seed=3, tensor_id=1)
    seed, m1, m2 = 11, 0x1234567, 0xFEDCBA9
    log("dual", shape, rr, cr)
    ro, co = fq.hadamard_quantize_dual(dev_bf16(bits), rr, m1, 1, cr, m2, 3, seed=seed)
    torch.cuda.synchronize()
    xf = host_f32(bits)
    wr = _oracle(xf, mx.ROW, rr, True, m1, seed, 1)
    wc = _oracle(xf, mx.COL, cr, True, m2, seed, 3)
    assert_bytes_equal(cpu(ro.codes), wr[0], "dual row codes")
    assert_bytes_equal(cpu(ro.scales), wr[1], "dual row scales")
    assert_bytes_equal(cpu(co.codes), wc[0], "dual col codes")
    assert_bytes_equal(cpu(co.scales), wc[1], "dual col scales")


def test_strided_input_rows():
    bits = synth.normal((64, 256), 1.0, seed=4, tensor_id=0)
    x = dev_bf16(bits)[:, :192]                     # ld 256, cols 192
    out = fq.quantize(x, axis=fq.ROW, rounding=fq.SR, seed=1, rng_stream=1, hadamard=True, mask=77)
    torch.cuda.synchronize()
    want = _oracle(host_f32(bits)[:, :192], mx.ROW, mx.SR, True, 77, 1, 1)
    assert_bytes_equal(cpu(out.codes), want[0], "strided codes")
    assert_bytes_equal(cpu(out.scales), want[1], "strided scales")


@pytest.mark.parametrize("rounding", [fq.RTN, fq.SR])
def test_quantizer_workload_full_size_row(rounding):
    """8192 x 4096, half N(0,1) / half Student-t(3), seed 0, GEMM-0 mask."""
    bits = synth.quantizer_tensor()["x"]
    mask = rng.sign_mask(0, 0)
    _check(bits, fq.ROW, rounding, True, mask=mask, seed=0, stream=1, what="c2-full")


@pytest.mark.parametrize("rounding", [fq.RTN, fq.SR])
def test_quantizer_workload_full_size_col(rounding):
    bits = synth.quantizer_tensor()["x"]
    _check(bits, fq.COL, rounding, True, mask=rng.sign_mask(0, 0), seed=0, stream=1, what="c2-full-col")


def test_col_axis_scales_at_odd_address():
    """Column-axis output whose scale pointer is not 4-byte aligned (scales
    are bytes; only codes must be 16-B aligned): same bytes as the oracle."""
    from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
    R, C = 256, 192
    bits = synth.normal_with_outliers((R, C), seed=3, tensor_id=0)
    x = dev_bf16(bits)
    codes = torch.empty((C, R // 2), dtype=torch.uint8, device="cuda")
    sbuf = torch.full((C * (R // 32) + 8,), 0xAB, dtype=torch.uint8, device="cuda")
    m = rng.sign_mask(3, 2)
    log("col axis, scales at offset 1")
    _check(fq.lib().fp4mx_hadamard_quantize(_ptr(x), R, C, C, fq.COL, fq.SR, m, 4, 3, _ptr(codes),
                                            sbuf.data_ptr() + 1, _stream()))
    torch.cuda.synchronize()
    wc, ws = mx.quantize(host_f32(bits), rounding=mx.SR, axis=mx.COL, sign_mask=m, seed=4, stream=3)
    got = cpu(sbuf)
    assert_bytes_equal(cpu(codes), wc, "codes")
    assert_bytes_equal(got[1:1 + ws.size].reshape(ws.shape), ws, "scales")
    assert got[0] == 0xAB and np.all(got[1 + ws.size:] == 0xAB)
