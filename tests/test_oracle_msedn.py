"""Pins for the oracle's unbiased NVFP4 backward quantizers: MS-EDEN and the
standard stochastic-rounding baseline (Quartet II page, Table 1, the EDEN
correction range, RHT_128 structure, unbiasedness)."""
import math

import numpy as np

from oracle import formats, msedn, nvfp4, rht


def _mse(d, ref):
    return float(np.mean((np.asarray(d, np.float64) - np.asarray(ref, np.float64)) ** 2) * 1e3)


def test_table1_ms_eden_and_sr(golden):
    """MSE x1e3 on N(0,1): MS-EDEN 9.8, SR 23.5 (one printed decimal, +-0.3)."""
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    x = np.random.default_rng(0).standard_normal((1024, 1024)).astype(np.float32)
    w = msedn.sign_mask128(0, 1)
    codes, sc, g, _ = msedn.msedn_quantize(x, w, seed=0, stream=5)
    y = msedn.rht128(x, w)          # MSE in the rotated basis (orthogonal: same as unrotated)
    got_eden = _mse(nvfp4.dequantize(codes, sc, g), y)
    c2, s2, g2 = msedn.sr_quantize(x, seed=0, stream=5)
    got_sr = _mse(nvfp4.dequantize(c2, s2, g2), x)
    assert abs(got_eden - want["ms_eden"]) < 0.3, got_eden
    assert abs(got_sr - want["sr"]) < 0.3, got_sr
    assert got_eden < got_sr / 2       # the page's "more than 2x lower"


def test_eden_correction_range(golden):
    lo, hi = (float(v) for v in golden("eden_s_range.txt")[0])
    x = np.random.default_rng(1).standard_normal((512, 1024)).astype(np.float32)
    _, _, S, _ = msedn.msedn_pass1(msedn.rht128(x, msedn.sign_mask128(3, 2)))
    assert S.min() >= lo and S.max() <= hi
    assert abs(float(np.mean(S)) - 1.0) < 0.02 and S.mean() > 1.0   # RTN loses energy on average


def test_rht128_is_signed_sylvester():
    words = msedn.sign_mask128(7, 0)
    s = msedn.signs128(words)
    H = rht.sylvester(128)
    x = np.random.default_rng(2).integers(-8, 9, (3, 128)).astype(np.float32)
    got = msedn.fwht128(x * s)
    assert np.array_equal(got, (x * s) @ H.T)                       # exact on small integers
    assert np.array_equal(H @ H.T, 128 * np.eye(128))
    assert msedn.INV_SQRT_128.view(np.uint32) == 0x3DB504F3
    # orthogonality and cancellation along the inner dimension
    a = np.random.default_rng(3).standard_normal((8, 256)).astype(np.float32)
    b = np.random.default_rng(4).standard_normal((5, 256)).astype(np.float32)
    ra, rb = msedn.rht128(a, words), msedn.rht128(b, words)
    assert np.allclose(ra.astype(np.float64) @ rb.T, a.astype(np.float64) @ b.T, rtol=1e-5, atol=1e-4)
    assert np.allclose(np.sum(ra.astype(np.float64) ** 2, axis=1), np.sum(a.astype(np.float64) ** 2, axis=1), rtol=1e-5)


def test_sign_words_differ_per_gemm_and_seed():
    ws = {tuple(msedn.sign_mask128(sd, g)) for sd in range(4) for g in range(3)}
    assert len(ws) == 12
    bits = sum(bin(v).count("1") for v in msedn.sign_mask128(0, 0))
    assert 40 < bits < 88


def test_e8m3_rne_brute_force():
    rs = np.random.default_rng(5)
    x = np.concatenate([rs.uniform(0, 1, 4000) * 10.0 ** rs.integers(-30, 30, 4000),
                        [0.0, 1.0, 1.0625, 1.03125, 1.09375, 15.5, 2.0 ** -130]]).astype(np.float32)
    got = msedn.e8m3_rne(x).astype(np.float64)
    for v, g in zip(x.astype(np.float64), got):
        if v == 0:
            assert g == 0
            continue
        if v < 2.0 ** -126:                      # fp32 subnormal: 2^20 encoding units = 2^-129
            step = 2.0 ** -129
        else:
            step = 2.0 ** (math.floor(math.log2(v)) - 3)
        lo = math.floor(v / step) * step
        cand = [lo, lo + step]
        d = [abs(c - v) for c in cand]
        if d[0] == d[1]:
            want = cand[0] if round(lo / step) % 2 == 0 else cand[1]
        else:
            want = cand[int(d[1] < d[0])]
        assert g == want, (v, g, want)


def test_e4m3_sr_probability_and_unbiased():
    grid = formats.E4M3_VALUES[:127]
    rs = np.random.default_rng(6)
    w = rs.uniform(0, 300, 64)
    w = np.concatenate([w, grid[:20], [2.0 ** -12, 447.0, 448.0]])
    u = np.arange(4096) / 4096.0
    for wi in w:
        c = msedn.e4m3_sr(np.full(u.shape, wi), u)
        vals = grid[c]
        assert np.all(vals <= max(wi, vals.min()) + 2 * (vals.max() - vals.min()) + 1e-12)
        assert abs(np.mean(vals) - min(wi, 448.0)) <= (grid[min(np.searchsorted(grid, wi), 126)] * 2 ** -12 + 1e-12)
        if wi in grid:
            assert np.all(vals == wi)


def test_range_exponent():
    for m in [1e-30, 0.7, 1.0, 255.9, 256.0, 256.1, 512.0, 3e5]:
        k = msedn.range_exponent(m)
        assert m * 2.0 ** -k <= 256.0 < m * 2.0 ** -(k - 1)
    assert msedn.range_exponent(0.0) == 0


def test_scale_sr_unbiased_over_seeds():
    """E over the SR seed of q * scale * g equals S * r (the EDEN correction)."""
    x = np.random.default_rng(8).standard_normal((8, 256)).astype(np.float32)
    w = msedn.sign_mask128(0, 1)
    y = msedn.rht128(x, w)
    q, vS, S, p = msedn.msedn_pass1(y)
    k = msedn.range_exponent(float(vS.max()))
    r = formats.e2m1_decode(q) * np.repeat(p, 16, axis=1)
    target = np.repeat(np.repeat(S, 8, axis=1), 16, axis=1) * r       # S * r per element
    acc = np.zeros_like(target)
    B = 400
    for sd in range(B):
        sc, g, _ = msedn.msedn_pass2(vS, seed=sd, stream=5, k=k)
        acc += formats.e2m1_decode(q) * np.repeat(formats.e4m3_decode(sc), 16, axis=1) * g
    mean = acc / B
    rel = np.linalg.norm(mean - target) / np.linalg.norm(target)
    one = np.linalg.norm(formats.e2m1_decode(q) * np.repeat(formats.e4m3_decode(msedn.msedn_pass2(vS, 0, 5, k=k)[0]), 16, axis=1) * g - target) / np.linalg.norm(target)
    assert rel < one / 8                                            # ~1/sqrt(B) shrinkage


def test_ms_eden_backward_gemm_unbiased():
    """Mean over seeds of the MS-EDEN product -> the exact product (1/B)."""
    rs = np.random.default_rng(9)
    a = rs.standard_normal((16, 256)).astype(np.float32)
    b = rs.standard_normal((12, 256)).astype(np.float32)
    exact = a.astype(np.float64) @ b.T.astype(np.float64)
    ests = []
    for sd in range(256):
        w = msedn.sign_mask128(sd, 1)
        qa = msedn.msedn_quantize(a, w, seed=sd, stream=5)[:3]
        qb = msedn.msedn_quantize(b, w, seed=sd, stream=6)[:3]
        ests.append(nvfp4.gemm_exact(*qa, *qb))
    ests = np.array(ests)

    def mse(B):
        m = ests[: (len(ests) // B) * B].reshape(-1, B, *exact.shape).mean(axis=1)
        return np.mean((m - exact) ** 2)
    e1, e16, e64 = mse(1), mse(16), mse(64)
    assert e16 < e1 / 8 and e64 < e1 / 25, (e1, e16, e64)


def test_sr_baseline_clip_free_and_unbiased():
    rs = np.random.default_rng(10)
    x = (rs.standard_normal((32, 64)) * np.exp(rs.uniform(-3, 3, (32, 1)))).astype(np.float32)
    # the 16/17 guard keeps |x / d| <= 6 without the clamp
    amax = np.float32(np.max(np.abs(x)))
    g = np.float32(amax / msedn.GUARD_D)
    blocks = x.reshape(32, 4, 16)
    t = (np.max(np.abs(blocks), -1) / np.float32(g * msedn.GUARD_C)).astype(np.float32)
    d = (formats.e4m3_decode(formats.e4m3_rne(t.astype(np.float64))).astype(np.float32) * g).astype(np.float32)
    assert np.max(np.abs(blocks / d[..., None])) <= 6.0 * (1 + 2 ** -22)
    acc = np.zeros(x.shape)
    B = 300
    for sd in range(B):
        acc += nvfp4.dequantize(*msedn.sr_quantize(x, seed=sd, stream=1))
    rel = np.linalg.norm(acc / B - x) / np.linalg.norm(x)
    one = np.linalg.norm(nvfp4.dequantize(*msedn.sr_quantize(x, seed=0, stream=1)) - x) / np.linalg.norm(x)
    assert rel < one / 8


def test_zero_rows_and_chunks():
    x = np.zeros((2, 256), np.float32)
    x[1, 128:] = np.random.default_rng(11).standard_normal(128)
    codes, sc, g, S = msedn.msedn_quantize(x, msedn.sign_mask128(0, 0), seed=0, stream=5)
    mag = formats.e2m1_decode(np.stack([codes & 7, codes >> 4 & 7], -1))    # rotated zeros may be -0
    assert np.all(mag[0] == 0) and np.all(sc[0] == 0) and np.all(S[0] == 1.0)
    assert np.all(mag[1, :64] == 0) and S[1, 0] == 1.0 and 0.9 < S[1, 1] < 1.1


def test_eden_s_scale_invariant_and_finite_for_huge_inputs():
    """S is taken on the power-of-two-scaled chunk: the same for x and
    2^j x, and finite when squares of the raw values would overflow fp32."""
    x = np.random.default_rng(14).standard_normal((4, 256)).astype(np.float32)
    w = msedn.sign_mask128(0, 0)
    S0 = msedn.msedn_pass1(msedn.rht128(x, w))[2]
    for j in (-100, 60, 100):
        Sj = msedn.msedn_pass1(msedn.rht128(np.ldexp(x, j).astype(np.float32), w))[2]
        assert np.array_equal(S0, Sj), j
    x[0, 3] = 1e30
    q, vS, S, p = msedn.msedn_pass1(msedn.rht128(x, w))
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(vS))
