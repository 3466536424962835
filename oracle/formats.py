"""Element and scale formats: E2M1 (FP4), E8M0 (MX scale), E4M3 (NVFP4 scale).

Test infrastructure (see the package docstring).

Sources:
* "Quartet II: Accurate LLM Pre-Training in NVFP4 ..." -- section "NVFP4
  Format and Standard Stochastic Rounding": the E2M1 value set
  {0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6}, E4M3 maximum 448, the SR rule
  (round up with probability (v-a)/(b-a)).
* "Bridging the Gap Between Promise and Performance for Microscaling FP4
  Quantization" -- "Formal Modeling of Microscaling Quantization Error" and
  "Shared Scale Quantization Effects": E2M1 is 1 sign, 2 exponent, 1 mantissa
  bit; E8M0 scales are pure powers of two over [2^-127, 2^127]; E4M3 range.
* "Quartet: Native FP4 Training ..." -- "The GPU Kernel Implementation",
  Stage 1: the group maximum is encoded as a power-of-two exponent.

Code layout of an E2M1 nibble: bit 3 is the sign, bits 2..0 index the
magnitude grid below (the OCP ordering, 2 exponent bits then 1 mantissa bit).
"""
from __future__ import annotations

import numpy as np

# Magnitudes indexed by the 3-bit code (0..7).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes -> float64 values (sign from bit 3)."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def _sign_bit(v: np.ndarray) -> np.ndarray:
    return (np.signbit(np.asarray(v, dtype=np.float32)).astype(np.uint8)) << 3


def _chunked(fn, x: np.ndarray, chunk: int) -> np.ndarray:
    """Apply an elementwise ``fn`` over a flattened array in fixed-size chunks
    (memory bound for the distance tables; no effect on the values)."""
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(0, flat.size, chunk):
        out[i:i + chunk] = fn(flat[i:i + chunk])
    return out.reshape(x.shape)


def e2m1_rtn(v: np.ndarray) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturating at 6.

    Plain definition: the distance from |v| to each of the eight grid points is
    computed exactly in float64 (v is float32, the grid is dyadic), the closest
    point wins, and of two equally close points the one with the even 3-bit
    code wins (IEEE round-half-to-even applied to the E2M1 encoding).  Values
    beyond 6 have 6 as their nearest point, so the rounding saturates.  The
    sign is kept, also for -0 and for negatives that round to zero.
    """
    v = np.asarray(v, dtype=np.float32)
    return _chunked(_e2m1_rtn_flat, v, 1 << 20)


def _e2m1_rtn_flat(v: np.ndarray) -> np.ndarray:
    # clamp first so that the float64 distances stay exact (6 is the nearest
    # grid point of every |v| >= 6 either way)
    a = np.minimum(np.abs(v.astype(np.float64)), 8.0)
    dist = np.abs(a[:, None] - E2M1_GRID[None, :])
    best = dist.min(axis=1)
    tie = dist == best[:, None]
    first = np.argmax(tie, axis=1)
    second_ok = np.zeros_like(tie[:, 0])
    has_next = first < 7
    second_ok[has_next] = tie[np.nonzero(has_next)[0], first[has_next] + 1]
    code = np.where(second_ok & (first % 2 == 1), first + 1, first).astype(np.uint8)
    return code.reshape(v.shape) | _sign_bit(v)


def e2m1_sr_carry(v: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Stochastic rounding onto the E2M1 grid driven by 32 random bits ``r``
    per element: the MXFP4 quantizer's backward rounding.

    The pages fix the rounding probability ("Quartet: Native FP4 Training
    ...", the SR step of the backward quantization; "NVFP4 Format and
    Standard Stochastic Rounding", Step 3): for a <= |v| < b with a, b
    adjacent grid points the magnitude becomes b with probability
    p = (|v|-a)/(b-a).  How the random bits realise that is this library's
    choice, at 22 bits, the fraction bits an fp32 significand keeps below an
    E2M1 gap of a normal value: the draw is u = (r >> 10) * 2^-22, and b is
    taken iff floor(p * 2^22) + (r >> 10) >= 2^22, i.e. the gap fraction
    truncated to 22 bits plus a 22-bit uniform carries.  P(b) =
    floor(p * 2^22) / 2^22: exactly p for every fp32 |v| >= 1, and for
    smaller |v| less than 2^-22 below p (a bias under 2^-23 of the scale).
    The sign is the sign of v (a negative value that rounds to 0 gives -0).
    Requires |v| <= 6 (the callers' scales guarantee no clipping).
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    if np.any(a > 6.0):
        raise ValueError("e2m1_sr_carry needs |v| <= 6")
    lo = np.minimum(np.searchsorted(E2M1_GRID, a, side="right") - 1, 7)   # grid[lo] <= a
    hi = np.minimum(lo + 1, 7)
    gap = np.where(hi > lo, E2M1_GRID[hi] - E2M1_GRID[lo], 1.0)
    p = np.where(hi > lo, (a - E2M1_GRID[lo]) / gap, 0.0)       # exact in float64
    t = np.floor(p * 2.0 ** 22).astype(np.uint64)               # exact: p < 1
    u22 = (np.asarray(r, dtype=np.uint32) >> np.uint32(10)).astype(np.uint64)
    up = (u22 + t) >= np.uint64(1 << 22)
    code = np.where(up, hi, lo).astype(np.uint8)
    return code | _sign_bit(v)


def e8m0_code(amax: np.ndarray) -> np.ndarray:
    """Shared MXFP4 scale exponent for a group with maximum magnitude ``amax``.

    Reading: the group maximum is encoded as a power of two (Quartet, Stage 1
    "Scale Factor Computation in E8M0") chosen so that the largest element
    lands in E2M1's top binade: X = 2^(floor(log2 amax) - 2), since E2M1's
    largest value 6 = 1.5 * 2^2.  The stored byte is that exponent plus the
    bias 127, clamped to E8M0's finite range [0, 254].  amax = 0 gives 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    floor_log2 = e.astype(np.int64) - 1
    code = floor_log2 - 2 + 127
    code = np.where(a == 0.0, 0, code)
    return np.clip(code, 0, 254).astype(np.uint8)


def e8m0_value(code: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2^(code-127) as float64 (0xFF is NaN)."""
    c = np.asarray(code).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


# --------------------------------------------------------------------------
# E4M3 (OCP "E4M3FN": bias 7, no infinities, max 448, subnormal step 2^-9).
# --------------------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    vals = np.zeros(128, dtype=np.float64)
    for c in range(128):
        e, m = c >> 3, c & 7
        if e == 0:
            vals[c] = (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    vals[127] = np.nan                      # 0x7F is NaN
    return vals


E4M3_VALUES = _e4m3_table()                 # magnitude by 7-bit code
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    mag = E4M3_VALUES[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Round to the nearest finite E4M3 value, ties to even code, saturating at 448.

    Plain definition over the 127 finite magnitudes; the sign bit is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    return _chunked(_e4m3_rne_flat, x, 1 << 16)


def _e4m3_rne_flat(x: np.ndarray) -> np.ndarray:
    a = np.minimum(np.abs(x), 512.0)       # keeps distances exact; 448 stays nearest
    grid = E4M3_VALUES[:127]
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1)
    tie = dist == best[:, None]
    first = np.argmax(tie, axis=1)
    has_next = first < 126
    second_ok = np.zeros_like(has_next)
    second_ok[has_next] = tie[np.nonzero(has_next)[0], first[has_next] + 1]
    code = np.where(second_ok & (first % 2 == 1), first + 1, first).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)
