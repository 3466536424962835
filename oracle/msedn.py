"""Unbiased NVFP4 quantizers for the backward pass: MS-EDEN and the standard
stochastic-rounding baseline.

Test infrastructure (see the package docstring).

Sources ("Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased
Gradient Estimation"):
* "NVFP4 Format and Standard Stochastic Rounding": the baseline Q_SR.  Global
  scale = amax / (6 * 16/17 * 448), group scale = RTN_FP8(group max /
  (global * 6 * 16/17)), elements = SR_FP4(x / (group scale * global)).
* "The EDEN Technique and Its Precision Bottleneck": S = <x, x> /
  <RHT(x), Q(RHT(x))> per rotation group.
* "MS-EDEN: Microscaling EDEN": RHT over chunks of 128 with one sign pattern
  per tensor; RTN NVFP4 with a clip factor s; S per 128-chunk; each group
  scale replaced by SR_FP8(S * group scale); the FP4 values stay RTN.
* "Kernel Speedups on NVIDIA Blackwell Hardware", post hoc range alignment:
  pass 1 quantizes against extended-range (E8M3) pseudo-scales and finds the
  global range and the correction factors; pass 2 reads only the scales,
  shifts them into the FP8 range, applies the correction and rounds to FP8
  stochastically.
* "Practical Performance of MS-EDEN", Table 1 (N(0,1), x 1e-3): SR 23.5,
  MS-EDEN 9.8; S in [0.94, 1.06] in practice (the pins in tests).

Readings taken (the pages leave these open):
* RHT_128: sign flip by a 128-bit mask (bit j of word j // 32 set <=> s_j =
  -1), radix-2 butterflies (a, b) -> (fl(a+b), fl(a-b)) on pairs (i, i+h) for
  h = 1, 2, ..., 64, then y = fl(t * c) with c = fl32(1/sqrt(128)).  Mask words
  0, 1 = lo32 / hi32 of splitmix64(seed ^ ((0x5200 + 2 g) << 32)), words 2, 3
  = lo32 / hi32 of splitmix64(seed ^ ((0x5201 + 2 g) << 32)) for GEMM id g.
* Post hoc range alignment with a power-of-two tensor scale, so that pass 1's
  FP4 codes stay exact after the shift:
    - pseudo-scale p = E8M3_RNE(fl(amax_b / s)): fp32 rounded to 4 significant
      bits (nearest, ties to even) on its encoding, exponent unbounded;
    - q_i = E2M1_RNE_sat(fl(y_i / p)) (q = sign only when p = 0);
    - r_i = val(q_i) * p (exact);
    - S = fl(num / den) per 128-chunk with num = sum fl(z_i^2), den =
      sum fl(z_i t_i), z = fl(y * 2^-E), t = fl(r * 2^-E), 2^E <= max|y| <
      2^(E+1) over the chunk (E = 0 for a zero chunk), both pairwise fp32
      trees in index order (S = 1 if den <= 0).  The power-of-two scaling
      leaves S unchanged mathematically and keeps the squares finite for any
      finite input;
    - v_g = fl(S * p_g); m = max over the tensor of v_g; tensor scale 2^k with
      k the least integer such that m * 2^-k <= 256 (k = 0 when m = 0);
    - group scale = SR_E4M3(fl32(v_g * 2^-k)) with u = (r >> 8) * 2^-24 from
      the counter generator at index row * (cols / 16) + group; the grid
      includes E4M3 subnormals; values >= 448 saturate (cannot happen: v <=
      256 * 2^-k * 2^k).
  E[scale * 2^k] = S * p_g, so E[q * scale * 2^k] = S * r: the EDEN
  correction applied in expectation, as the pages describe.
* Baseline Q_SR: c = fl32(6 * 16/17), D = fl32(c * 448), g = fl(amax / D),
  s16 = E4M3_RNE(fl(amax_b / fl(g * c))), d = fl(s16 * g), v = fl(x / d)
  (clamped to |v| <= 6 against fp32 rounding), q = SR_E2M1(v) with u from
  the generator at index row * cols + col.
* Inputs must be finite.
"""
from __future__ import annotations

import numpy as np

from . import formats, rng

CHUNK = 128
GROUP = 16
INV_SQRT_128 = np.float32(1.0 / np.sqrt(128.0))      # 0x3DB504F3
RANGE_CAP = 256.0


# ---------------------------------------------------------------------------
# RHT over 128-element chunks
# ---------------------------------------------------------------------------

def sign_mask128(seed: int, gemm_id: int) -> list[int]:
    """Four 32-bit words of the 128-element sign pattern of GEMM ``gemm_id``."""
    a = rng.splitmix64((seed ^ ((0x5200 + 2 * gemm_id) << 32)) & rng.M64)
    b = rng.splitmix64((seed ^ ((0x5201 + 2 * gemm_id) << 32)) & rng.M64)
    return [a & 0xFFFFFFFF, a >> 32, b & 0xFFFFFFFF, b >> 32]


def signs128(words: list[int]) -> np.ndarray:
    return np.array([-1.0 if (words[j // 32] >> (j % 32)) & 1 else 1.0 for j in range(CHUNK)],
                    dtype=np.float32)


def fwht128(t: np.ndarray) -> np.ndarray:
    """Unnormalised FWHT over the last axis (length 128), float32 butterflies."""
    t = np.array(t, dtype=np.float32, copy=True)
    h = 1
    while h < CHUNK:
        for i in range(CHUNK):
            if i & h:
                continue
            a = t[..., i].copy()
            b = t[..., i + h].copy()
            t[..., i] = a + b
            t[..., i + h] = a - b
        h *= 2
    return t


def rht128(x: np.ndarray, words: list[int]) -> np.ndarray:
    """y = c * H (s * x) per 128-chunk of the last axis, in float32."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    assert shp[-1] % CHUNK == 0
    blocks = x.reshape(shp[:-1] + (shp[-1] // CHUNK, CHUNK))
    y = fwht128(blocks * signs128(words)) * INV_SQRT_128
    return y.astype(np.float32).reshape(shp)


# ---------------------------------------------------------------------------
# Small exact helpers
# ---------------------------------------------------------------------------

def e8m3_rne(x: np.ndarray) -> np.ndarray:
    """Round non-negative float32 values to 4 significant bits (3 fraction
    bits), nearest with ties to even, on the fp32 encoding (exponent range of
    fp32, hence 'E8M3')."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFFF + ((b >> 20) & 1)) & ~np.uint64(0xFFFFF)
    return b.astype(np.uint32).view(np.float32)


def _pairwise(v: np.ndarray) -> np.ndarray:
    """Pairwise fp32 sum over the last axis (a power of two): pairs (2i, 2i+1),
    then pairs of those sums, down to one."""
    s = v.astype(np.float32)
    while s.shape[-1] > 1:
        s = (s[..., 0::2] + s[..., 1::2]).astype(np.float32)
    return s[..., 0]


def e4m3_sr(w: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Stochastic rounding of non-negative values onto the E4M3 grid
    (subnormals included, saturating at 448): the upper neighbour b is taken
    iff u < (w - a) / (b - a)."""
    w = np.minimum(np.asarray(w, dtype=np.float64), formats.E4M3_MAX)
    grid = formats.E4M3_VALUES[:127]
    lo = np.searchsorted(grid, w, side="right") - 1
    lo = np.minimum(lo, 126)
    hi = np.minimum(lo + 1, 126)
    ga, gb = grid[lo], grid[hi]
    p = np.where(hi > lo, (w - ga) / np.where(hi > lo, gb - ga, 1.0), 0.0)
    return np.where(np.asarray(u, dtype=np.float64) < p, hi, lo).astype(np.uint8)


def _pack(q: np.ndarray) -> np.ndarray:
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------------------
# MS-EDEN (post hoc range alignment)
# ---------------------------------------------------------------------------

def msedn_pass1(y: np.ndarray, s: float = 6.0):
    """Pass 1 on the rotated tensor y [R, C] (C % 128 == 0).

    Returns (q codes [R, C] uint8 (sign in bit 3), v = fl(S * p) [R, C/16]
    float32, S [R, C/128] float32, p [R, C/16] float32)."""
    y = np.asarray(y, dtype=np.float32)
    R, C = y.shape
    g16 = y.reshape(R, C // GROUP, GROUP)
    amax_b = np.max(np.abs(g16), axis=-1).astype(np.float32)
    p = e8m3_rne((amax_b / np.float32(s)).astype(np.float32))
    pe = p[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(pe > 0, (g16 / np.where(pe > 0, pe, 1)).astype(np.float32),
                     np.where(np.signbit(g16), np.float32(-0.0), np.float32(0.0)))
    q = formats.e2m1_rtn(v.astype(np.float32))
    r = (formats.e2m1_decode(q).astype(np.float32) * pe).astype(np.float32)
    yc = y.reshape(R, C // CHUNK, CHUNK)
    rc = r.reshape(R, C // CHUNK, CHUNK)
    # S is invariant under scaling the chunk by a power of two: the sums are
    # taken on y * 2^-E, r * 2^-E with 2^E <= max|y| < 2^(E+1), so no square
    # overflows (exact scaling whenever nothing under- or overflows)
    E = chunk_exponent(np.max(np.abs(yc), axis=-1))
    ys = np.ldexp(yc, -E[..., None]).astype(np.float32)
    rsc = np.ldexp(rc, -E[..., None]).astype(np.float32)
    num = _pairwise((ys * ys).astype(np.float32))
    den = _pairwise((ys * rsc).astype(np.float32))
    with np.errstate(divide="ignore", invalid="ignore"):
        S = np.where(den > 0, (num / np.where(den > 0, den, 1)).astype(np.float32), np.float32(1.0))
    vS = (np.repeat(S, CHUNK // GROUP, axis=-1) * p).astype(np.float32)
    return q.reshape(R, C), vS, S.astype(np.float32), p


def chunk_exponent(m: np.ndarray) -> np.ndarray:
    """floor(log2 m) for m > 0 (fp32 subnormals included), 0 for m = 0."""
    f, e = np.frexp(np.asarray(m, dtype=np.float64))
    return np.where(np.asarray(m) > 0, e - 1, 0).astype(np.int64)


def range_exponent(m: float) -> int:
    """Least integer k with m * 2^-k <= 256 (0 for m = 0)."""
    if m <= 0:
        return 0
    f, e = np.frexp(np.float64(m))          # m = f * 2^e, f in [0.5, 1)
    lg = e - 1 if f == 0.5 else e           # ceil(log2 m)
    return int(lg - 8)


def msedn_pass2(vS: np.ndarray, seed: int, stream: int, row_ids=None, k: int | None = None):
    """Pass 2: tensor scale 2^k and the stochastically rounded E4M3 scales.

    ``row_ids`` are the rows' indices in the full output operand (for sampled
    rows); ``k`` overrides the range exponent (taken from the full tensor)."""
    vS = np.asarray(vS, dtype=np.float32)
    R, G = vS.shape
    if k is None:
        k = range_exponent(float(np.max(vS)) if vS.size else 0.0)
    w = np.ldexp(vS, -k).astype(np.float32)
    rows = np.arange(R, dtype=np.uint64) if row_ids is None else np.asarray(row_ids, dtype=np.uint64)
    idx = rows[:, None] * np.uint64(G) + np.arange(G, dtype=np.uint64)[None, :]
    u = rng.uniform24(rng.bits(seed, stream, idx))
    codes = e4m3_sr(w, u)
    return codes, np.float32(np.ldexp(np.float32(1.0), k)), k


def msedn_quantize(x: np.ndarray, words: list[int], seed: int, stream: int, s: float = 6.0,
                   row_ids=None, k: int | None = None):
    """MS-EDEN of x [R, C] along rows (128-chunks along C).

    Returns (codes [R, C/2] uint8, scales [R, C/16] E4M3 uint8, g float32,
    S [R, C/128])."""
    y = rht128(x, words)
    q, vS, S, _ = msedn_pass1(y, s)
    sc, g, _ = msedn_pass2(vS, seed, stream, row_ids=row_ids, k=k)
    return _pack(q), sc, g, S


def msedn_range_exponent(x: np.ndarray, words: list[int], s: float = 6.0) -> int:
    """k of the whole tensor (needed when quantizing sampled rows)."""
    _, vS, _, _ = msedn_pass1(rht128(x, words), s)
    return range_exponent(float(np.max(vS)))


# ---------------------------------------------------------------------------
# Baseline: standard NVFP4 stochastic rounding (16/17 guard)
# ---------------------------------------------------------------------------

GUARD_C = np.float32(6.0 * 16.0 / 17.0)
GUARD_D = np.float32(GUARD_C * np.float32(448.0))


def sr_quantize(x: np.ndarray, seed: int, stream: int):
    """Q_SR of x [R, C] (groups of 16 along rows).

    Tensor scale with the 16/17 guard, E4M3 group scales by RNE, then each
    v = fl(x / fl(s16 g)), clamped to [-6, 6], rounded stochastically onto
    the E2M1 grid ("Quartet II ...", "NVFP4 Format and Standard Stochastic
    Rounding").  The pages fix the rounding probability p = (|v|-a)/(b-a);
    the random bits realise it by the same 22-bit carry rule as the MXFP4
    backward quantizer (``formats.e2m1_sr_carry`` on the counter hash at
    index row * C + col): unbiased for every |v| >= 1, short of p by less
    than 2^-22 below 1.

    Returns (codes [R, C/2] uint8, scales [R, C/16] E4M3 uint8, g float32)."""
    a = np.asarray(x, dtype=np.float32)
    R, C = a.shape
    amax = np.float32(np.max(np.abs(a))) if a.size else np.float32(0)
    g = np.float32(amax / GUARD_D)
    blocks = a.reshape(R, C // GROUP, GROUP)
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    gc = np.float32(g * GUARD_C)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(gc > 0, (amax_b / gc).astype(np.float32), np.float32(0))
    s_code = formats.e4m3_rne(t.astype(np.float64))
    d = (formats.e4m3_decode(s_code).astype(np.float32) * g).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d > 0, (blocks / np.where(d > 0, d, 1)).astype(np.float32),
                     np.where(np.signbit(blocks), np.float32(-0.0), np.float32(0.0)))
    v = np.clip(v, np.float32(-6.0), np.float32(6.0)).reshape(R, C)
    idx = (np.arange(R, dtype=np.uint64)[:, None] * np.uint64(C)
           + np.arange(C, dtype=np.uint64)[None, :])
    q = formats.e2m1_sr_carry(v, rng.bits(seed, stream, idx))
    return _pack(q), s_code, g
