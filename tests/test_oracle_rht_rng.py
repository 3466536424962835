"""Pins for the oracle's randomized Hadamard transform and counter RNG."""
import numpy as np
import scipy.linalg

from oracle import rht, rng


def test_fwht_is_sylvester_hadamard():
    # FWHT of the unit vectors gives the columns of H (exact: no rounding)
    H = rht.fwht32(np.eye(32, dtype=np.float32)).T.astype(np.float64)
    assert np.array_equal(H, scipy.linalg.hadamard(32))
    assert np.array_equal(H @ H.T, 32 * np.eye(32))        # H H^T = 32 I


def test_kronecker_recursion():
    H2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    Hk = H2
    for n in (4, 8, 16, 32, 64, 128, 256):
        Hk = np.kron(H2, Hk)
        assert np.array_equal(Hk, rht.sylvester(n))
        assert np.array_equal(Hk @ Hk.T, n * np.eye(n))


def test_normalisation_constant():
    c = rht.INV_SQRT_G
    assert c.view(np.uint32) == 0x3E3504F3
    # nearest float32 to 1/sqrt(32): compare squared distances exactly in fp64
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(1))]
    err = [abs(float(x) ** 2 * 32 - 1) for x in cands]
    assert err[1] < err[0] and err[1] < err[2]


def test_rht_exact_on_integers_and_signs():
    rs = np.random.default_rng(2)
    x = rs.integers(-50, 50, (16, 64)).astype(np.float32)
    mask = 0xA5C3_1F07
    y = rht.rht32(x, mask)
    s = np.array([-1 if (mask >> j) & 1 else 1 for j in range(32)], dtype=np.float64)
    H = scipy.linalg.hadamard(32).astype(np.float64)
    ref = (x.reshape(16, 2, 32).astype(np.float64) * s) @ H.T   # exact integers
    ref32 = (ref.astype(np.float32) * rht.INV_SQRT_G).astype(np.float32).reshape(16, 64)
    assert np.array_equal(y, ref32)


def test_rht_orthogonal_roundtrip_and_cancellation():
    rs = np.random.default_rng(3)
    a = rs.standard_normal((8, 256)).astype(np.float32)
    b = rs.standard_normal((8, 256)).astype(np.float32)
    mask = rng.sign_mask(7, 1)
    ya, yb = rht.rht32(a, mask), rht.rht32(b, mask)
    # norm preserved
    assert np.allclose(np.linalg.norm(ya, axis=1), np.linalg.norm(a, axis=1), rtol=1e-6)
    # inverse: x = s * (H y) / sqrt(32)
    back = rht.rht32(ya, 0) * rht.signs(mask).reshape(1, 32).repeat(8, 0).reshape(-1)[:256]
    assert np.allclose(back, a, atol=4e-6 * np.abs(a).max())
    # rotations cancel in the inner product
    assert np.allclose(ya.astype(np.float64) @ yb.T.astype(np.float64),
                       a.astype(np.float64) @ b.T.astype(np.float64), atol=1e-4)


def test_rng_published_vectors(golden):
    rows = golden("rng_vectors.txt")
    sm = [r for r in rows if r[0] == "splitmix64_state0"][0][1:]
    state = 0
    for want in sm:
        assert rng.splitmix64(state) == int(want, 16)
        state = (state + rng.GOLDEN_GAMMA) & rng.M64
    for r in rows:
        if r[0] == "fmix32":
            assert rng.fmix32(int(r[1], 16)) == int(r[2], 16)
            assert int(rng.fmix32(np.array([int(r[1], 16)], dtype=np.uint32))[0]) == int(r[2], 16)


def test_rng_uniformity_and_streams():
    idx = np.arange(1 << 18, dtype=np.uint64)
    u1 = rng.uniform24(rng.bits(0, 1, idx))
    u2 = rng.uniform24(rng.bits(0, 2, idx))
    assert abs(u1.mean() - 0.5) < 0.003
    counts = np.bincount((u1 * 16).astype(int), minlength=16)
    exp = len(u1) / 16
    assert ((counts - exp) ** 2 / exp).sum() < 50          # chi2(15) 99.99% ~ 44
    assert abs(np.corrcoef(u1, u2)[0, 1]) < 0.01
    assert abs(np.corrcoef(u1[:-1], u1[1:])[0, 1]) < 0.01
    # 64-bit indices use the high word
    hi = rng.bits(0, 1, idx + np.uint64(1 << 32))
    assert not np.array_equal(hi, rng.bits(0, 1, idx))
    assert rng.sign_mask(0, 0) != rng.sign_mask(0, 1)
