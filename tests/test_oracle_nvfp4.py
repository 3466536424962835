"""Pins for the oracle's NVFP4 forward variant (Table 1 of the Quartet II page)."""
import numpy as np

from oracle import formats, nvfp4


def test_table1_rtn_and_four_over_six(golden):
    want = {r[0]: float(r[1]) for r in golden("nvfp4_table1_mse.txt")}
    x = np.random.default_rng(0).standard_normal((1024, 1024)).astype(np.float32)
    got = {}
    for name, use46 in (("rtn", False), ("rtn_46", True)):
        d = nvfp4.dequantize(*nvfp4.quantize46(x, use46))
        got[name] = np.mean((d - x) ** 2) * 1e3
    # the page prints one decimal: hold to +-0.3e-3
    for k in got:
        assert abs(got[k] - want[k]) < 0.3, (k, got[k], want[k])
    assert got["rtn_46"] < got["rtn"]


def test_four_over_six_block_choice_and_ranges():
    rs = np.random.default_rng(1)
    x = (rs.standard_normal((64, 256)) * rs.uniform(0.01, 10, (64, 1))).astype(np.float32)
    c6, s6, g = nvfp4.quantize46(x, False)
    c46, s46, g2 = nvfp4.quantize46(x, True)
    assert g == g2 == np.float32(np.float32(np.abs(x).max()) / np.float32(1536))
    d6 = nvfp4.dequantize(c6, s6, g).reshape(64, 16, 16)
    d46 = nvfp4.dequantize(c46, s46, g).reshape(64, 16, 16)
    xb = x.reshape(64, 16, 16).astype(np.float64)
    e6 = ((d6 - xb) ** 2).sum(axis=2)
    e46 = ((d46 - xb) ** 2).sum(axis=2)
    assert np.all(e46 <= e6 * (1 + 1e-5) + 1e-30)
    # group scales stay well inside E4M3 (<= 384 by construction, < 448 max)
    assert formats.e4m3_decode(s46).max() <= 384 * 1.07
    # some blocks pick each candidate
    assert np.any(s46 != s6) and np.any(s46 == s6)


def test_zero_and_tiny_blocks():
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, :16] = 1.0
    x[1, 16] = -1e-30
    c, s, g = nvfp4.quantize46(x, True)
    d = nvfp4.dequantize(c, s, g)
    assert np.all(d[0, 16:] == 0) and np.all(d[1, :16] == 0)
    assert np.allclose(d[0, :16], 1.0)


def test_fp8_staging_range_and_accuracy():
    rs = np.random.default_rng(2)
    a = rs.standard_normal((32, 256)).astype(np.float32)
    b = (rs.standard_normal((48, 256)) * 0.02).astype(np.float32)
    qa, qb = nvfp4.quantize46(a), nvfp4.quantize46(b)
    st, e = nvfp4.fp8_stage(qa[0], qa[1])
    assert np.abs(st).max() <= 360
    exact = nvfp4.gemm_exact(*qa, *qb)
    staged = nvfp4.gemm_fp8_staged(*qa, *qb)
    rel = np.linalg.norm(staged - exact) / np.linalg.norm(exact)
    # E4M3 staging rounds q*s16 (up to 6 significant bits) to 4 bits: 2-4% on
    # the affected elements, a few percent on the product
    assert rel < 4e-2
    # exact when the staged products need no rounding: s16 powers of two
    q = formats.e2m1_rtn(rs.standard_normal((4, 64)).astype(np.float32))
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    scales = formats.e4m3_rne(np.ldexp(1.0, rs.integers(-3, 4, (4, 4))))
    st2, e2 = nvfp4.fp8_stage(codes, scales)
    full = st2 * np.ldexp(1.0, np.repeat(e2, 32, axis=1))
    assert np.array_equal(full, nvfp4.dequantize(codes, scales, 1.0))


def test_fp8_staging_exhaustive_against_torch():
    """Every (E2M1 code, positive finite E4M3 scale of its group, scale of the
    other group in the 32-block) staged as the library's FP8 GEMM expects,
    against an independent route: the block exponent from a brute-force search
    for each scale's power of two, the product q * s16 * 2^-e_blk formed
    exactly (at most 6 significant bits, so exact in fp32), and the E4M3
    rounding done by torch's float8_e4m3fn conversion."""
    import torch
    scales = np.arange(0x7F, dtype=np.uint8)                  # 0 .. 0x7E: +0 and every positive finite E4M3
    sa, sb = np.meshgrid(scales, scales, indexing="ij")
    sa, sb = sa.ravel(), sb.ravel()                           # 16129 scale pairs, one block row each
    rows = sa.size
    nib = np.arange(16, dtype=np.uint8)
    half = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)    # the 16 codes of one 16-group, packed
    codes = np.tile(np.concatenate([half, half]), (rows, 1))  # [rows, 16] bytes = 32 elements
    sc = np.stack([sa, sb], axis=1)                           # [rows, 2] E4M3 bytes
    got_b, got_e = nvfp4.fp8_stage_bytes(codes, sc)

    # independent route
    def pow2_floor(s):
        """largest e with 2^e <= s, by search (None for 0)."""
        if s == 0:
            return None
        e = -30
        while 2.0 ** (e + 1) <= s:
            e += 1
        return e
    val = {int(c): float(formats.e4m3_decode(np.array([c]))[0]) for c in scales}
    pe = {c: pow2_floor(v) for c, v in val.items()}
    e_blk = np.empty(rows, np.int64)
    for i, (a, b) in enumerate(zip(sa, sb)):
        es = [e for e in (pe[int(a)], pe[int(b)]) if e is not None]
        e_blk[i] = max(es) - 5 if es else 0
    assert np.array_equal(got_e[:, 0], e_blk)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    qv = np.where(nib & 8, -grid[nib & 7], grid[nib & 7])       # the 16 code values
    s16 = np.stack([np.vectorize(val.get)(sa), np.vectorize(val.get)(sb)], axis=1).astype(np.float64)
    prod = qv[None, None, :] * s16[:, :, None] * np.ldexp(1.0, -e_blk)[:, None, None]
    p32 = prod.astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), prod)        # exact before the FP8 rounding
    want = torch.from_numpy(p32.reshape(rows, 32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got_b, want)
    # the staged magnitudes stay inside E4M3's range: at most 6 * 1.875 * 2^5
    assert np.abs(prod).max() == 360.0
