"""Pins for the oracle's Quartet II graph with re-quantized saved operands
(Quartet II page: "The Complete Quartet II Computation Graph", Table 1)."""
from fractions import Fraction

import numpy as np

from oracle import formats, msedn, nvfp4, quartet2 as q2


def _bf16(x):
    from fp4_microscaled_quantized_amd import synth
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


def _saved(shape, seed, std=1.0):
    x = _bf16(np.random.default_rng(seed).standard_normal(shape) * std)
    return nvfp4.quantize46(x, True), x


def test_dequantize32_is_the_rounded_exact_product():
    (codes, scales, g), _ = _saved((8, 64), 1, 0.37)
    got = q2.dequantize32(codes, scales, g)
    q = np.empty((8, 64))
    q[:, 0::2] = formats.e2m1_decode(codes & 0xF)
    q[:, 1::2] = formats.e2m1_decode(codes >> 4)
    s = np.repeat(formats.e4m3_decode(scales), 16, axis=1)
    for i in range(0, 8, 3):
        for j in range(0, 64, 7):
            exact = Fraction(float(q[i, j])) * Fraction(float(s[i, j])) * Fraction(float(g))
            assert got[i, j] == np.float32(float(exact)), (i, j)


def test_requantize_error_matches_table1(golden):
    """MS-EDEN on re-quantized N(0,1) operands keeps the page's error level
    (Table 1: 9.8e-3 relative to the unit variance) and beats SR by > 2x."""
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    (c, s, g), _ = _saved((512, 1024), 2)
    words = msedn.sign_mask128(4, 1)
    v = q2.dequantize32(c, s, g)
    yt = msedn.rht128(np.ascontiguousarray(v.T), words).astype(np.float64)
    rc, rs, rg, S = q2.requantize(c, s, g, words, seed=4, stream=6)
    rel = np.mean((nvfp4.dequantize(rc, rs, rg) - yt) ** 2) / np.mean(yt ** 2) * 1e3
    assert abs(rel - want["ms_eden"]) < 0.6
    sc, ss, sg = msedn.sr_quantize(np.ascontiguousarray(v.T), seed=4, stream=6)
    rel_sr = np.mean((nvfp4.dequantize(sc, ss, sg) - v.T) ** 2) / np.mean(v.astype(np.float64) ** 2) * 1e3
    assert rel < rel_sr / 2
    assert 0.94 <= S.min() and S.max() <= 1.06


def test_requantize_sampled_rows_match_full():
    (c, s, g), _ = _saved((256, 96), 3)
    words = msedn.sign_mask128(2, 2)
    full = q2.requantize(c, s, g, words, seed=2, stream=8)
    k = q2.requant_range_exponent(c, s, g, words)
    rows = np.array([0, 17, 95])
    part = q2.requantize(c, s, g, words, seed=2, stream=8, row_ids=rows, k=k)
    assert np.array_equal(part[0], full[0][rows]) and np.array_equal(part[1], full[1][rows])
    assert part[2] == full[2]


def test_linear_bwd_unbiased():
    x = _bf16(np.random.default_rng(5).standard_normal((128, 64)))
    w = _bf16(np.random.default_rng(6).standard_normal((128, 64)))
    dy = _bf16(np.random.default_rng(7).standard_normal((128, 128)))
    _, ctx = q2.linear_fwd(x, w)
    ex_dx, ex_dw = q2.expected_grads(dy, ctx)
    dxs, dws = [], []
    for sd in range(96):
        dx, dw = q2.linear_bwd(dy, ctx, sd)
        dxs.append(dx)
        dws.append(dw)
    for ests, ex in ((np.array(dxs), ex_dx), (np.array(dws), ex_dw)):
        def err(B):
            mm = ests[: (len(ests) // B) * B].reshape(-1, B, *ex.shape).mean(axis=1)
            return np.mean((mm - ex) ** 2)
        e1, e16, e48 = err(1), err(16), err(48)
        assert e16 < e1 / 8 and e48 < e1 / 20


def test_backward_close_to_exact_gradient():
    x = _bf16(np.random.default_rng(8).standard_normal((128, 256)))
    w = _bf16(np.random.default_rng(9).standard_normal((128, 256)) * 0.02)
    dy = _bf16(np.random.default_rng(10).standard_normal((128, 128)) * 1e-3)
    _, ctx = q2.linear_fwd(x, w)
    dx, dw = q2.linear_bwd(dy, ctx, 1)
    e = dy.astype(np.float64)
    tdx, tdw = e @ w.astype(np.float64), e.T @ x.astype(np.float64)
    assert np.linalg.norm(dx - tdx) / np.linalg.norm(tdx) < 0.25
    assert np.linalg.norm(dw - tdw) / np.linalg.norm(tdw) < 0.25
