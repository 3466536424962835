"""Pins for the oracle's codecs (E2M1, E8M0, E4M3) against the pages and
independent routes (numpy's round-half-even, torch's float8_e4m3fn)."""
import math

import numpy as np
import pytest
import torch

from oracle import formats

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_e2m1_grid_matches_pages(golden):
    grid = np.array([float(r[0]) for r in golden("e2m1_grid.txt")])
    assert np.array_equal(formats.E2M1_GRID, grid)
    vals = formats.e2m1_decode(np.arange(16))
    assert np.array_equal(vals[:8], grid)
    assert np.array_equal(vals[8:], -grid)
    consts = {r[0]: float(r[1]) for r in golden("format_constants.txt")}
    assert grid.max() == consts["e2m1_max"]


def _rtn_textbook(v):
    """Independent route: round-half-even (np.rint) at each E2M1 binade's step."""
    a = np.abs(v.astype(np.float64))
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.rint(a / step) * step
    r = np.minimum(r, 6.0)
    # E2M1 codes for the grid values
    lut = {g: i for i, g in enumerate(formats.E2M1_GRID)}
    code = np.array([lut[x] for x in r.tolist()], dtype=np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def test_e2m1_rtn_ties_and_saturation():
    cases = {0.0: 0, 0.24: 0, 0.25: 0, 0.26: 1, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4,
             3.5: 6, 5.0: 6, 5.01: 7, 7.0: 7, 7.99: 7, 1e30: 7}
    v = np.array(list(cases), dtype=np.float32)
    assert list(formats.e2m1_rtn(v)) == list(cases.values())
    assert list(formats.e2m1_rtn(-v)) == [c | 8 for c in cases.values()]
    assert formats.e2m1_rtn(np.float32(-0.0)) == 8


def test_e2m1_rtn_dense_sweep_vs_textbook():
    # every float32 with exponent in [2^-3, 2^3) at mantissa stride 97, plus
    # every grid point and midpoint and their fp32 neighbours
    e = np.arange(124, 130, dtype=np.uint32)
    m = np.arange(0, 1 << 23, 97, dtype=np.uint32)
    bits = ((e[:, None] << 23) | m[None, :]).reshape(-1)
    v = bits.view(np.float32)
    pts = np.concatenate([formats.E2M1_GRID, (formats.E2M1_GRID[1:] + formats.E2M1_GRID[:-1]) / 2])
    pts = pts.astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(10))])
    v = np.concatenate([v, near, -near]).astype(np.float32)
    assert np.array_equal(formats.e2m1_rtn(v), _rtn_textbook(v))


def _rtn_textbook_vec(v):
    """_rtn_textbook without the Python-level lookup (for large sweeps)."""
    a = np.abs(v.astype(np.float64))
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.minimum(np.rint(a / step) * step, 6.0)
    code = np.searchsorted(formats.E2M1_GRID, r).astype(np.uint8)
    assert np.array_equal(formats.E2M1_GRID[code], r)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def test_e2m1_rtn_exhaustive_over_fp32():
    """Every fp32 input, both signs: each of the 2^23 mantissas of every
    exponent in [2^-4, 2^4) (all grid points, midpoints and their neighbours
    lie there), and every exponent outside that range at the mantissas where
    a piecewise-constant rule could change (0, 1, the middle, the maximum),
    with subnormals and zeros."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in range(123, 131):
        for sgn in (0, 1):
            bits = (np.uint32(sgn) << np.uint32(31)) | (np.uint32(e) << np.uint32(23)) | mant
            v = bits.view(np.float32)
            assert np.array_equal(formats.e2m1_rtn(v), _rtn_textbook_vec(v)), (e, sgn)
    edge_m = np.array([0, 1, 1 << 22, (1 << 23) - 1], dtype=np.uint32)
    ex = np.array([e for e in range(0, 255) if not 123 <= e <= 130], dtype=np.uint32)
    bits = ((ex[:, None] << np.uint32(23)) | edge_m[None, :]).reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(1 << 31)])
    v = bits.view(np.float32)
    assert np.array_equal(formats.e2m1_rtn(v), _rtn_textbook_vec(v))


def test_e2m1_sr_carry_exact_over_a_complete_stratum():
    # The decision depends on the top 22 bits of r only.  Enumerating all 2^22
    # of them, the fraction that rounds up is p truncated to 22 bits: exactly
    # p for |v| >= 1 and for smaller |v| whose gap position has <= 22 bits, so
    # the decoded mean is |v| to the last bit there ...
    k = np.arange(1 << 22, dtype=np.uint64)
    r = ((k << np.uint64(10)) | np.uint64(0x2A5)).astype(np.uint32)   # the low 10 bits are ignored
    for v in [1.3, 2.7, 5.1, 4.0, 5.999999, 1.0000001, 6.0, -3.3, 0.625, 0.2578125, 0.5]:
        vf = np.float32(v)
        dec = formats.e2m1_decode(formats.e2m1_sr_carry(np.full(k.shape, vf), r))
        assert dec.sum() / float(1 << 22) == float(vf), v
    # ... and below 1 the mean falls short of |v| by less than 2^-22 of the gap
    for v in [0.7, 0.3, 0.26, 0.1, 1e-3, 3e-7]:
        vf = np.float32(v)
        dec = formats.e2m1_decode(formats.e2m1_sr_carry(np.full(k.shape, vf), r))
        short = float(vf) - dec.sum() / float(1 << 22)
        assert 0.0 <= short < 0.5 * 2.0 ** -22, (v, short)


def test_e2m1_sr_carry_orientation_and_sign():
    # the largest draw rounds every interior point up, the smallest none
    v = np.array([0.1, 0.75, 1.2, 2.5, 4.5, -0.1, -3.5, 1e-30, -0.0, 0.0], dtype=np.float32)
    hi = formats.e2m1_decode(formats.e2m1_sr_carry(v, np.full(v.shape, 0xFFFFFFFF, np.uint32)))
    lo = formats.e2m1_decode(formats.e2m1_sr_carry(v, np.zeros(v.shape, np.uint32)))
    assert list(hi) == [0.5, 1.0, 1.5, 3.0, 6.0, -0.5, -4.0, 0.0, 0.0, 0.0]
    assert list(lo) == [0.0, 0.5, 1.0, 2.0, 4.0, -0.0, -3.0, 0.0, 0.0, 0.0]
    # sign bit follows v, also for values that round to zero and for -0
    q = formats.e2m1_sr_carry(v, np.zeros(v.shape, np.uint32))
    assert list(q >> 3) == [0, 0, 0, 0, 0, 1, 1, 0, 1, 0]
    # a gap position below 2^-22 never rounds up; 2^-22 itself does with the largest draw
    assert formats.e2m1_sr_carry(np.float32(2.0 ** -24), np.uint32(0xFFFFFFFF)) == 0
    assert formats.e2m1_sr_carry(np.float32(2.0 ** -23), np.uint32(0xFFFFFFFF)) == 1
    assert formats.e2m1_sr_carry(np.float32(2.0 ** -23), np.uint32(0xFFFFFBFF)) == 0


def test_e2m1_sr_carry_unbiased_monte_carlo():
    rs = np.random.default_rng(6)
    v = (rs.random(64) * 12 - 6).astype(np.float32)
    n = 20000
    r = rs.integers(0, 1 << 32, (n, 64), dtype=np.uint64).astype(np.uint32)
    q = formats.e2m1_decode(formats.e2m1_sr_carry(np.broadcast_to(v, (n, 64)), r))
    mean = q.mean(axis=0)
    sd = q.std(axis=0) / np.sqrt(n) + 1e-12
    assert np.all(np.abs(mean - v) < 5 * sd + 1e-9)


def test_e8m0_code_properties():
    rs = np.random.default_rng(0)
    # normal fp32 maxima across the whole exponent range
    bits = (rs.integers(1, 255, 20000, dtype=np.uint32) << 23) | rs.integers(0, 1 << 23, 20000, dtype=np.uint32)
    amax = bits.view(np.float32).astype(np.float64)
    code = formats.e8m0_code(amax).astype(np.int64)
    X = np.ldexp(1.0, code - 127)
    inner = (code > 0) & (code < 254)
    r = amax[inner] / X[inner]
    # the largest element lands in E2M1's top binade [4, 8)
    assert np.all((r >= 4) & (r < 8))
    # library route: frexp exponent
    _, e = np.frexp(amax)
    assert np.array_equal(code, np.clip(e - 1 - 2 + 127, 0, 254))
    assert formats.e8m0_code(np.array([0.0, 6.0, 8.0, 1e-45, 3.4028235e38])).tolist() == [0, 127, 128, 0, 252]


def test_e8m0_code_exhaustive_over_exponents():
    """Every fp32 exponent (subnormals included) at the smallest, a middle and
    the largest mantissa, against frexp's exponent: code = clamp(floor(log2
    amax) - 2 + 127, 0, 254)."""
    ex = np.arange(0, 255, dtype=np.uint32)
    mant = np.array([1, 1 << 22, (1 << 23) - 1], dtype=np.uint32)
    bits = ((ex[:, None] << np.uint32(23)) | mant[None, :]).reshape(-1)
    amax = bits.view(np.float32).astype(np.float64)
    _, e = np.frexp(amax)
    want = np.clip(e - 1 - 2 + 127, 0, 254)
    assert np.array_equal(formats.e8m0_code(amax).astype(np.int64), want)


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = formats.e4m3_decode(np.arange(256))
    fin = ~np.isnan(b)
    assert np.array_equal(np.isnan(ours), np.isnan(b))
    assert np.array_equal(ours[fin], b[fin])


def test_e4m3_rne_matches_torch(golden):
    consts = {r[0]: float(r[1]) for r in golden("format_constants.txt")}
    assert formats.E4M3_VALUES[126] == consts["e4m3_max"]
    rs = np.random.default_rng(1)
    x = np.concatenate([
        rs.standard_normal(20000) * 30,
        np.exp(rs.uniform(np.log(1e-4), np.log(440), 20000)),
        formats.E4M3_VALUES[:127],
        (formats.E4M3_VALUES[:126] + formats.E4M3_VALUES[1:127]) / 2,       # ties
    ])
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3_rne(x), t)
    assert formats.e4m3_rne(np.array([1000.0]))[0] == 126            # saturates
