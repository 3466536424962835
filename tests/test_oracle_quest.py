"""Pins for the oracle's QuEST forward quantizer and the Quartet backward in the
forward-rotated basis (Quartet page: "The Forward-Pass Quantization: QuEST in
Detail", the clipping-mask correction and inverse Hadamard, "The Complete
Quartet Algorithm")."""
import math

import numpy as np
import pytest

from oracle import formats, mx, quest, rht, rng


def _bf16(x):
    from fp4_microscaled_quantized_amd import synth
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


# --------------------------- the clip factor -------------------------------

def _q_scaled(x, c):
    """RTN of clamp(|x|, 0, c) onto the E2M1 grid scaled by c/6 (nearest point)."""
    grid = quest.E2M1_GRID * (c / 6.0)
    a = np.minimum(np.abs(x), c)
    return grid[np.argmin(np.abs(a[..., None] - grid), axis=-1)]


@pytest.mark.parametrize("c", [1.0, 2.0, 2.9, 4.0, 5.0])
def test_gaussian_mse_closed_form_vs_quadrature(c):
    from scipy import integrate
    grid = quest.E2M1_GRID * (c / 6.0)
    f = lambda x: (x - grid[np.argmin(np.abs(min(x, c) - grid))]) ** 2 * math.exp(-x * x / 2) \
        / math.sqrt(2 * math.pi)
    pts = list((quest.E2M1_GRID[1:] + quest.E2M1_GRID[:-1]) / 2 * (c / 6.0)) + [c]
    val = 2 * (integrate.quad(f, 0, c, points=pts, limit=200, epsabs=1e-14)[0]
               + integrate.quad(f, c, np.inf, epsabs=1e-14)[0])
    assert abs(quest.gaussian_mse(c) - val) < 1e-9 * val


def test_gaussian_mse_monte_carlo():
    x = np.random.default_rng(5).standard_normal(2_000_000)
    for c in (2.0, 2.92):
        e = (np.abs(x) - _q_scaled(x, c)) ** 2
        se = e.std() / math.sqrt(e.size)
        assert abs(e.mean() - quest.gaussian_mse(c)) < 4 * se


def test_optimal_clip_is_the_minimum():
    from scipy import optimize
    c = quest.optimal_clip()
    assert 1.0 <= c <= 5.0
    f = quest.gaussian_mse
    grid = np.linspace(1, 5, 801)
    assert f(c) <= min(f(float(g)) for g in grid) + 1e-15
    r = optimize.minimize_scalar(f, bounds=(1, 5), method="bounded", options={"xatol": 1e-10})
    assert abs(r.x - c) < 1e-6
    assert f(c - 1e-3) > f(c) and f(c + 1e-3) > f(c)


def test_library_default_clip_is_the_optimum():
    import fp4_microscaled_quantized_amd as fq
    c = quest.optimal_clip()
    assert abs(fq.QUEST_CLIP - c) < 1e-6
    assert quest.gaussian_mse(fq.QUEST_CLIP) - quest.gaussian_mse(c) < 1e-12


# --------------------------- the quantizer ----------------------------------

def test_mse_ranking_matches_the_page():
    """Gaussian data: QuEST has the lowest MSE, SR (AbsMax) the highest, RTN
    (AbsMax) in between (the ranking reported with page 1's Table 2)."""
    x = _bf16(np.random.default_rng(0).standard_normal((512, 1024)))
    m = rng.sign_mask(3, 0)
    y = rht.rht32(x, m).astype(np.float64)
    cq, sq, _ = quest.quest_quantize(x, m, quest.optimal_clip())
    e_q = np.mean((mx.dequantize(cq, sq) - y) ** 2)
    e_r = np.mean((mx.dequantize(*mx.quantize(x, rounding=mx.RTN, sign_mask=m)) - y) ** 2)
    s = mx.quantize(x, rounding=mx.SR, sign_mask=m, seed=1, stream=1)
    e_s = np.mean((mx.dequantize(*s) / 0.75 - y) ** 2)
    assert e_q < 0.98 * e_r < e_s


@pytest.mark.parametrize("scale", [1.0, 1e30, 1e-30, 3e-3])
def test_sigma_and_threshold_against_numpy(scale):
    x = _bf16(np.random.default_rng(2).standard_normal((64, 256)) * scale)
    m, c = rng.sign_mask(1, 0), 2.5
    sig, T = quest.group_sigma_threshold(x, m, c)
    y = rht.rht32(x, m).astype(np.float64).reshape(64, 8, 32)
    ref = y.std(axis=2)
    assert np.all(np.abs(sig - ref) <= 4e-6 * ref)
    assert np.all(np.abs(T - c * ref) <= 5e-6 * c * ref)


def test_scales_and_mask_against_fp64():
    x = _bf16(np.random.default_rng(4).standard_normal((128, 512)) * 0.02)
    m, c = rng.sign_mask(9, 0), quest.optimal_clip()
    codes, sc, mask = quest.quest_quantize(x, m, c)
    y = rht.rht32(x, m).astype(np.float64).reshape(128, 16, 32)
    T64 = c * y.std(axis=2)
    lg = np.log2(T64)
    safe = np.abs(lg - np.round(lg)) > 1e-5
    want = np.floor(lg).astype(np.int64) + 125
    assert np.all(sc.astype(np.int64)[safe] == want[safe])
    bits = quest.unpack_mask(mask, 512).reshape(128, 16, 32)
    lim = np.minimum(T64, 6.0 * np.ldexp(1.0, sc.astype(np.int64) - 127))
    far = np.abs(np.abs(y) - lim[..., None]) > 1e-5 * lim[..., None]
    assert np.array_equal(bits[far], (np.abs(y) > lim[..., None])[far])
    assert 0.0005 < bits.mean() < 0.05


def test_mask_covers_every_saturated_element():
    """With a power-of-two scale X the grid ends at 6 X while T / X lies in
    [4, 8): an element beyond 6 X is clipped by the saturating rounding even
    when it is below T, and its gradient must be masked like a clamped one."""
    x = _bf16(np.random.default_rng(12).standard_t(4, (256, 512)))
    m, c = rng.sign_mask(13, 0), quest.optimal_clip()
    codes, sc, mask = quest.quest_quantize(x, m, c)
    y = rht.rht32(x, m).astype(np.float64).reshape(256, 16, 32)
    _, T = quest.group_sigma_threshold(x, m, c)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127)
    bits = quest.unpack_mask(mask, 512).reshape(256, 16, 32)
    beyond_grid = np.abs(y) > 6.0 * X[..., None]
    beyond_T = np.abs(y) > T.astype(np.float64)[..., None]
    # both kinds of clipping occur, and T > 6 X in a good share of the groups
    assert beyond_grid.any() and beyond_T.any()
    assert 0.2 < np.mean(T > 6.0 * X) < 0.7
    assert np.all(bits[beyond_grid]) and np.all(bits[beyond_T])
    assert np.array_equal(bits, beyond_grid | beyond_T)
    # an element that is not masked is represented without saturation:
    # its magnitude code is below 6, or it rounded to 6 from at most 6 X
    q = mx.unpack(codes).reshape(256, 16, 32) & 7
    assert np.all(np.abs(y)[(q == 7) & ~bits] <= 6.0 * X[..., None].repeat(32, 2)[(q == 7) & ~bits])


def test_clipped_groups_reduce_to_mx_rtn():
    """Where a group clips, its scale encodes T = max of the clamped group, so
    its codes are MX RTN (no transform) of the clamped group."""
    x = _bf16(np.random.default_rng(6).standard_t(3, (96, 256)))
    m, c = rng.sign_mask(2, 0), 2.0
    codes, sc, mask = quest.quest_quantize(x, m, c)
    y = rht.rht32(x, m)
    _, T = quest.group_sigma_threshold(x, m, c)
    Tb = np.repeat(T, 32, axis=1)
    cl = np.where(np.abs(y) > Tb, np.copysign(Tb, y), y).astype(np.float32)
    rc, rs = mx.quantize(cl, rounding=mx.RTN, hadamard=False)
    clips = quest.unpack_mask(mask, 256).reshape(96, 8, 32).any(axis=2)
    assert clips.mean() > 0.3
    assert np.array_equal(sc[clips], rs[clips])
    q, rq = mx.unpack(codes).reshape(96, 8, 32), mx.unpack(rc).reshape(96, 8, 32)
    assert np.array_equal(q[clips], rq[clips])


def test_power_of_two_scale_invariance():
    x = _bf16(np.random.default_rng(7).standard_normal((32, 256)))
    m, c = rng.sign_mask(4, 0), quest.optimal_clip()
    c0, s0, m0 = quest.quest_quantize(x, m, c)
    for k in (-40, 13, 60):
        c1, s1, m1 = quest.quest_quantize(np.ldexp(x, k), m, c)
        assert np.array_equal(c0, c1) and np.array_equal(m0, m1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_degenerate_groups():
    x = np.zeros((32, 96), np.float32)
    x[1, :32] = -0.0
    x[2, 32] = 3.0                 # one nonzero input in a block: constant rotated group
    x[3, 64:] = np.inf             # non-finite group
    x[4] = _bf16(np.random.default_rng(1).standard_normal(96))
    codes, sc, mask = quest.quest_quantize(x, 0, 2.9)
    q = mx.unpack(codes)
    bits = quest.unpack_mask(mask, 96)
    assert np.all(q[0] == 0) and np.all(sc[0] == 0) and not bits[0].any()
    assert np.all(sc[1] == 0) and not bits[1].any()
    # constant group: sigma = 0, T = 0, every element clipped to +0 and masked
    assert sc[2, 1] == 0 and np.all(q[2, 32:64] == 0) and bits[2, 32:64].all()
    assert sc[3, 2] == 0xFF and np.all(q[3, 64:] == 0) and not bits[3, 64:].any()
    assert np.all(sc[4] > 100)


def test_clip_large_means_no_mask_and_scale_from_T():
    x = _bf16(np.random.default_rng(8).standard_normal((16, 128)))
    codes, sc, mask = quest.quest_quantize(x, 0, 1e3)
    assert not quest.unpack_mask(mask, 128).any()
    sig, T = quest.group_sigma_threshold(x, 0, 1e3)
    assert np.array_equal(sc.astype(np.int64), quest._floor_log2(T) + 125)


def test_scale_code_saturates_at_254():
    """A threshold beyond the E8M0 range gives scale 254 (never a wrapped
    byte or the 0xFF marker), finite codes and no mask bits."""
    rs = np.random.default_rng(14)
    x = _bf16(rs.standard_normal((8, 64)) * 1e36)     # transform sums stay finite
    for clip in (8.0, 1e3, 3.0e38):
        codes, sc, mask = quest.quest_quantize(x, 0, clip)
        _, T = quest.group_sigma_threshold(x, 0, clip)
        want = np.where(np.isinf(T), 254, np.minimum(quest._floor_log2(np.where(np.isinf(T), 1, T)) + 125, 254))
        assert np.array_equal(sc.astype(np.int64), want)
        assert np.all(sc <= 254) and not quest.unpack_mask(mask, 64).any()
        y = rht.rht32(x, 0).astype(np.float64)
        deq = mx.dequantize(codes, sc)
        # no sign flips: every nonzero code has the sign of its element
        nz = deq != 0
        assert np.all(np.sign(deq[nz]) == np.sign(y[nz]))


# --------------------------- backward pieces --------------------------------

def test_dequantize32_exact_and_bf16_representable():
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)        # every nibble pair
    for e in (0, 1, 100, 127, 200, 251):
        sc = np.full((8, 2), e, np.uint8)
        v = quest.dequantize32(codes, sc)
        ref = mx.dequantize(codes, sc)
        assert np.array_equal(v.astype(np.float64), ref)
        assert np.array_equal(_bf16(v), v)
    assert np.all(np.isnan(quest.dequantize32(codes, np.full((8, 2), 255, np.uint8))[:, 1:]))


def test_inverse_rht_against_matrix_inverse():
    m = rng.sign_mask(11, 0)
    B = rht.sylvester(32) / math.sqrt(32.0) * rht.signs(m)[None, :].astype(np.float64)
    y = np.random.default_rng(3).standard_normal((5, 64))
    want = np.linalg.solve(B, y.reshape(10, 32).T).T.reshape(5, 64)
    assert np.allclose(quest.inverse_rht64(y, m), want, rtol=1e-12, atol=1e-12)
    x = np.random.default_rng(4).standard_normal((5, 64)).astype(np.float32)
    assert np.allclose(quest.inverse_rht64(rht.rht32(x, m), m), x, rtol=0, atol=2e-6)


def test_unmask_zeroes_clipped_entries_before_inverse():
    c = np.random.default_rng(5).standard_normal((4, 64))
    bits = np.random.default_rng(6).random((4, 64)) < 0.2
    mask = np.packbits(bits, axis=1, bitorder="little")
    got = quest.unmask_inverse_rht(c, mask, 0x1234)
    assert np.allclose(got, quest.inverse_rht64(np.where(bits, 0.0, c), 0x1234), atol=1e-12)
    # the mask removes exactly the masked coordinates of the rotated gradient
    back = rht.rht32(got.astype(np.float32), 0x1234)
    assert np.allclose(back[bits], 0, atol=1e-6)


def test_requantize_unbiased_over_seeds():
    a = _bf16(np.random.default_rng(9).standard_normal((64, 96)))
    ac, as_ = mx.quantize(a, rounding=mx.RTN, sign_mask=0)
    d = quest.dequantize32(ac, as_)
    m = rng.sign_mask(5, 1)
    target = rht.rht32(np.ascontiguousarray(d.T), m).astype(np.float64)   # [96, 64]
    acc = np.zeros_like(target)
    B = 200
    for s in range(B):
        rc, rs = quest.requantize(ac, as_, m, seed=s, stream=2)
        acc += mx.dequantize(rc, rs) / 0.75
    err = np.linalg.norm(acc / B - target) / np.linalg.norm(target)
    assert err < 0.05
    one = np.linalg.norm(mx.dequantize(*quest.requantize(ac, as_, m, 0, 2)) / 0.75 - target)
    assert err < one / np.linalg.norm(target) / 6


# --------------------------- the linear layer -------------------------------

def _layer(seed=0, m=64, n=96, k=128, w_std=1.0):
    rs = np.random.default_rng(seed)
    x = _bf16(rs.standard_normal((m, k)))
    w = _bf16(rs.standard_normal((n, k)) * w_std)
    dy = _bf16(rs.standard_normal((m, n)))
    return x, w, dy


def test_linear_fwd_close_to_exact():
    x, w, _ = _layer()
    y, ctx = quest.linear_fwd(x, w, seed=3, clip=quest.optimal_clip())
    ex = x.astype(np.float64) @ w.astype(np.float64).T
    ry = np.linalg.norm(y - ex) / np.linalg.norm(ex)
    y_mx, _ = mx.linear_fwd(x, w, seed=3, want_ctx=False)
    assert ry < 0.2 and ry < np.linalg.norm(y_mx - ex) / np.linalg.norm(ex)
    assert quest.unpack_mask(ctx["mx"], 128).any()


def test_linear_bwd_unbiased():
    x, w, dy = _layer(1)
    _, ctx = quest.linear_fwd(x, w, seed=5, clip=quest.optimal_clip())
    ex_dx, ex_dw = quest.expected_grads(dy, ctx)
    dxs, dws = [], []
    for s in range(128):
        c2 = dict(ctx, seed=s)
        # the forward masks of seed 5 stay; only the backward draws change
        dx, dw = _bwd_with_fwd_mask(dy, c2, 5)
        dxs.append(dx)
        dws.append(dw)
    for ests, ex in ((np.array(dxs), ex_dx), (np.array(dws), ex_dw)):
        def err(B):
            mm = ests[: (len(ests) // B) * B].reshape(-1, B, *ex.shape).mean(axis=1)
            return np.mean((mm - ex) ** 2)
        e1, e16, e64 = err(1), err(16), err(64)
        assert e16 < e1 / 8 and e64 < e1 / 25


def _bwd_with_fwd_mask(dy, ctx, fwd_seed):
    """linear_bwd with the backward draws of ctx['seed'] and the inverse
    rotation of the forward seed (test helper: decouples the two)."""
    seed = ctx["seed"]
    g0 = rng.sign_mask(fwd_seed, 0)
    g1, g2 = rng.sign_mask(seed, 1), rng.sign_mask(seed, 2)
    dyq = mx.quantize(dy, rounding=mx.SR, axis=mx.ROW, sign_mask=g1, seed=seed, stream=1)
    dyt = mx.quantize(dy, rounding=mx.SR, axis=mx.COL, sign_mask=g2, seed=seed, stream=3)
    wt = quest.requantize(*ctx["wq"], g1, seed, 2)
    xt = quest.requantize(*ctx["xq"], g2, seed, 4)
    return (quest.unmask_inverse_rht(mx.gemm(*dyq, *wt, alpha=mx.ALPHA_BWD), ctx["mx"], g0),
            quest.unmask_inverse_rht(mx.gemm(*dyt, *xt, alpha=mx.ALPHA_BWD), ctx["mw"], g0))


def test_linear_bwd_matches_helper_at_the_forward_seed():
    x, w, dy = _layer(2)
    _, ctx = quest.linear_fwd(x, w, seed=7, clip=2.5)
    a = quest.linear_bwd(dy, ctx)
    b = _bwd_with_fwd_mask(dy, ctx, 7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_expected_grads_without_clipping_is_the_dequantized_product():
    """No element clipped: E[dX] = dY W~ with W~ = H^-1(deq(W_q)) the forward
    weights in the original basis (linearity of H^-1), close to dY W."""
    x, w, dy = _layer(3)
    _, ctx = quest.linear_fwd(x, w, seed=1, clip=8.0)
    assert not quest.unpack_mask(ctx["mx"], 128).any()
    ex_dx, ex_dw = quest.expected_grads(dy, ctx)
    g0 = rng.sign_mask(1, 0)
    wt = quest.inverse_rht64(mx.dequantize(*ctx["wq"]), g0)
    assert np.allclose(ex_dx, dy.astype(np.float64) @ wt, rtol=1e-10, atol=1e-10)
    d = dy.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(ex_dx - d) / np.linalg.norm(d) < 0.3
