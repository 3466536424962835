"""QuEST forward quantization (MXFP4, clipping mask) and the Quartet backward
in the forward-rotated basis (re-quantized saved operands, mask correction,
inverse Hadamard).

Test infrastructure (see the package docstring).

Sources ("Quartet: Native FP4 Training Can Be Optimal for Large Language
Models"):
* "The Forward-Pass Quantization: QuEST in Detail": groups of 32 along the
  GEMM inner dimension after the Hadamard transform; per-group standard
  deviation sigma (about the group mean); a clip factor c in [1, 5] that
  minimises RMSE(c)^2 = E_{x~N(0,1)}[(x - Q(clamp(x, -c, c)))^2]; group scale
  c sigma / 6; x_q = RTN(clamp(x, -c sigma, c sigma) / s); a mask bit per
  element that is set when the element was clipped.  The same section calls
  the minimisation analytic.
* "The GPU Kernel Implementation: Two-Stage Fused Design", Stage 1: on the
  forward pass the value that is encoded as the E8M0 power of two is the one
  the clip factor determines; the mask bit is set iff |x| > c sigma (under
  the page's scale c sigma / 6, c sigma is also where the grid ends; see the
  mask reading below).
* "The Hadamard Transform: Why It Is Necessary and How It Is Implemented",
  inverse Hadamard and clipping-mask correction: dx = 16/9 H^-1(dx_q o M_x),
  and the same for dW with M_w; the mask removes the gradient of clipped
  elements.
* "The Complete Quartet Algorithm: Step-by-Step Execution": the forward saves
  {X_q, W_q, M_x, M_w} (no bf16 activations); the backward dequantizes W_q and
  X_q, transposes them, applies the randomized Hadamard transform along the
  backward GEMM's inner dimension (same seed for both operands of a GEMM),
  quantizes with SR(3/4 .), multiplies, then applies the mask and H^-1.

Readings taken (the pages leave these open or disagree):
* The clip factor.  The printed objective takes the expectation over
  x ~ N(0,1) with the scale c/6 (so c maps to the grid maximum 6); its minimum
  over [1, 5] is one constant, c* = 2.92247508... (``optimal_clip``), and the
  per-group work is sigma and T = fl(c* sigma).  This is the "analytic"
  minimisation; a caller may pass any other c > 0.
* sigma is the population standard deviation about the group mean, evaluated
  in fp32 on the group scaled by 2^-E, 2^E <= max|y| < 2^(E+1) (E = 0 for a
  zero group), so that squares neither overflow nor underflow:
  mu = fl(tree(z) / 32), var = fl(tree(fl(fl(z - mu)^2)) / 32),
  sigma_z = fl(sqrt(var)), T_z = fl(c sigma_z); tree = adjacent pairs summed
  level by level in index order.  T = fl(T_z 2^E) (may be +inf, then nothing
  clips).
* The E8M0 scale encodes T by the rule of the MX path (floor(log2 T) - 2):
  code = max(floor(log2 T_z) + E + 125, 0), code 0 when T_z = 0, at most 254
  (a T_z that overflowed to inf gives 254).  With this rule QuEST's MSE on
  N(0,1) is below AbsMax RTN's, the ranking the page reports; taking the
  scale from min(amax, T) instead would invert it.
* Clamp: an element with |y| > T becomes sign(y) T, others are kept;
  v = fl(clamped * 2^(127 - code)); code = E2M1 RNE, saturating, sign bit
  kept.  A group with sigma = 0 (for example one nonzero input in a Hadamard
  block, which makes the rotated group constant) has T = 0: every nonzero
  element is clipped to 0 and masked.
* Mask.  The page's scale c sigma / 6 maps [-c sigma, c sigma] onto the grid's
  range, and the mask flags the elements that were clipped.  With a
  power-of-two scale X the grid ends at 6 X, and T / X lies in [4, 8), so when
  T > 6 X the elements with 6 X < |y| <= T are clipped by the saturating
  rounding instead of the clamp.  Reading: the effective clip is min(T, 6 X)
  and the mask bit is |y| > min(T, 6 X) (compared exactly; 6 X beyond the
  fp32 range clips nothing).
* A non-finite group (after the transform) gets scale 0xFF, element codes 0
  and mask bits 0, as on the MX path.
* The page multiplies dx_q by M_x while saying the mask zeroes the gradient of
  the clipped elements, whose bit is 1; the stated purpose is taken: the
  correction multiplies by (1 - M).
* H^-1 is the inverse of the forward rotation y = c H (s o x): x = s o (c H y).
  The backward masks and streams are those of the MX linear layer: dY rows
  SR (mask of GEMM 1, stream 1), dY^T SR (GEMM 2, stream 3), W_q re-quantized
  along N (GEMM 1, stream 2), X_q along M (GEMM 2, stream 4).
* Dequantized MXFP4 values q 2^(e-127) are exact in fp32 and in bf16 (at most
  two significant bits; 0xFF is NaN, products beyond the fp32 range are inf).

Mask layout: uint8 [rows, cols / 8]; element j of a row is bit j % 8 of byte
j // 8.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats, mx, rht, rng

GROUP = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# ---------------------------------------------------------------------------
# The clip factor: minimum of the Gaussian RMSE objective over [1, 5]
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def gaussian_mse(c: float) -> float:
    """E[(x - Q_c(clamp(x, -c, c)))^2] for x ~ N(0,1), Q_c = RTN onto the
    E2M1 grid scaled by c/6, in closed form.

    On an interval [a, b] where Q_c is the constant g:
    int (x - g)^2 phi = [Phi - x phi]_a^b + 2 g [phi]_a^b + g^2 [Phi]_a^b;
    beyond c the element is clipped to c: int_c^inf (x - c)^2 phi =
    (1 + c^2)(1 - Phi(c)) - c phi(c).  Symmetric, so twice the half line.
    """
    s = c / 6.0
    g = E2M1_GRID * s
    edges = [0.0] + list((E2M1_GRID[1:] + E2M1_GRID[:-1]) / 2.0 * s) + [c]
    tot = 0.0
    for i, gi in enumerate(g):
        a, b = edges[i], edges[i + 1]
        m2 = (_Phi(b) - b * _phi(b)) - (_Phi(a) - a * _phi(a))
        m1 = -_phi(b) + _phi(a)
        m0 = _Phi(b) - _Phi(a)
        tot += m2 - 2.0 * gi * m1 + gi * gi * m0
    tot += (1.0 + c * c) * (1.0 - _Phi(c)) - c * _phi(c)
    return 2.0 * tot


def optimal_clip() -> float:
    """argmin of gaussian_mse over [1, 5]: a grid of step 1e-3, then golden
    section search on the bracketing interval (float64)."""
    cs = np.linspace(1.0, 5.0, 4001)
    vals = [gaussian_mse(float(c)) for c in cs]
    i = int(np.argmin(vals))
    lo, hi = float(cs[max(i - 1, 0)]), float(cs[min(i + 1, len(cs) - 1)])
    r = (math.sqrt(5.0) - 1.0) / 2.0
    a, b = lo, hi
    c1, c2 = b - r * (b - a), a + r * (b - a)
    f1, f2 = gaussian_mse(c1), gaussian_mse(c2)
    for _ in range(200):
        if f1 < f2:
            b, c2, f2 = c2, c1, f1
            c1 = b - r * (b - a)
            f1 = gaussian_mse(c1)
        else:
            a, c1, f1 = c1, c2, f2
            c2 = a + r * (b - a)
            f2 = gaussian_mse(c2)
        if b - a < 1e-13:
            break
    return 0.5 * (a + b)


# ---------------------------------------------------------------------------
# QuEST quantization of one operand (groups along rows)
# ---------------------------------------------------------------------------

def _tree(v: np.ndarray) -> np.ndarray:
    """fp32 sum over the last axis (length 32): adjacent pairs, level by level."""
    v = np.asarray(v, dtype=np.float32)
    while v.shape[-1] > 1:
        v = (v[..., 0::2] + v[..., 1::2]).astype(np.float32)
    return v[..., 0]


def _floor_log2(v: np.ndarray) -> np.ndarray:
    """floor(log2 v) for positive finite float32 v (subnormals included)."""
    _, ex = np.frexp(np.asarray(v, dtype=np.float32))
    return ex.astype(np.int64) - 1


def quest_quantize(x: np.ndarray, sign_mask: int, clip: float, hadamard: bool = True):
    """QuEST MXFP4 quantization of x [R, C] (float32 holding bf16 values)
    along rows, after the block-32 RHT with ``sign_mask``.

    Returns (codes [R, C/2] uint8, scales [R, C/32] uint8, mask [R, C/8] uint8).
    """
    a = np.asarray(x, dtype=np.float32)
    R, C = a.shape
    if C % GROUP:
        raise ValueError("the grouped dimension must be a multiple of 32")
    y = rht.rht32(a, sign_mask) if hadamard else a.copy()
    g = y.reshape(R, C // GROUP, GROUP)
    with np.errstate(invalid="ignore", over="ignore"):
        finite = np.all(np.isfinite(g), axis=2)
        gs = np.where(finite[..., None], g, np.float32(0)).astype(np.float32)
        amax = np.max(np.abs(gs), axis=2)
        E = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1)), 0)
        z = np.ldexp(gs, -E[..., None]).astype(np.float32)
        mu = (_tree(z) * np.float32(0.03125)).astype(np.float32)
        d = (z - mu[..., None]).astype(np.float32)
        var = (_tree((d * d).astype(np.float32)) * np.float32(0.03125)).astype(np.float32)
        sig = np.sqrt(var).astype(np.float32)
        tz = (np.float32(clip) * sig).astype(np.float32)
        ok = (tz > 0) & np.isfinite(tz)
        code = np.where(ok, _floor_log2(np.where(ok, tz, 1)) + E + 125, 0)
        code = np.where(np.isinf(tz), 254, np.clip(code, 0, 254))
        T = np.ldexp(tz, E).astype(np.float32)
        clipped = np.abs(gs) > T[..., None]
        cl = np.where(clipped, np.copysign(np.broadcast_to(T[..., None], gs.shape), gs), gs)
        inv = np.ldexp(np.float32(1.0), (127 - code).astype(np.int32)).astype(np.float32)
        v = (cl.astype(np.float32) * inv[..., None]).astype(np.float32)
        # the effective clip is min(T, 6 X): beyond 6 X the E2M1 grid saturates
        lim = np.minimum(T.astype(np.float64), 6.0 * np.ldexp(1.0, code.astype(np.int64) - 127))
        masked = np.abs(gs.astype(np.float64)) > lim[..., None]
    q = formats.e2m1_rtn(v)
    q = np.where(finite[..., None], q, 0).astype(np.uint8).reshape(R, C)
    clipped = np.where(finite[..., None], masked, False).reshape(R, C)
    code = np.where(finite, code, 255).astype(np.uint8)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    mask = np.packbits(clipped, axis=1, bitorder="little")
    return packed, code, mask


def group_sigma_threshold(x: np.ndarray, sign_mask: int, clip: float):
    """(sigma, T) per group as fp32 arrays [R, C/32], by the same steps as
    ``quest_quantize`` (finite groups)."""
    y = rht.rht32(np.asarray(x, dtype=np.float32), sign_mask)
    R, C = y.shape
    g = y.reshape(R, C // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    E = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1)), 0)
    z = np.ldexp(g, -E[..., None]).astype(np.float32)
    mu = (_tree(z) * np.float32(0.03125)).astype(np.float32)
    d = (z - mu[..., None]).astype(np.float32)
    var = (_tree((d * d).astype(np.float32)) * np.float32(0.03125)).astype(np.float32)
    sig = np.sqrt(var).astype(np.float32)
    with np.errstate(over="ignore"):
        T = np.ldexp((np.float32(clip) * sig).astype(np.float32), E).astype(np.float32)
    return np.ldexp(sig, E).astype(np.float32), T


def unpack_mask(mask: np.ndarray, cols: int) -> np.ndarray:
    """[R, C/8] bytes -> bool [R, C]."""
    return np.unpackbits(np.asarray(mask, dtype=np.uint8), axis=1, bitorder="little",
                         count=cols).astype(bool)


# ---------------------------------------------------------------------------
# Backward helpers
# ---------------------------------------------------------------------------

def dequantize32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 operand -> float32 values (exact; 0xFF -> NaN, beyond range -> inf)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return mx.dequantize(codes, scales).astype(np.float32)


def requantize(codes: np.ndarray, scales: np.ndarray, sign_mask: int, seed: int, stream: int,
               rounding: int = mx.SR):
    """Dequantize an MXFP4 operand [R, C] (groups along C), transpose it and
    quantize it again along R with the RHT: the transposed operand [C, R]."""
    return mx.quantize(dequantize32(codes, scales), rounding=rounding, axis=mx.COL,
                       sign_mask=sign_mask, seed=seed, stream=stream)


def inverse_rht64(y: np.ndarray, sign_mask: int) -> np.ndarray:
    """x = s o (c H y) per 32-block of the last axis, in float64."""
    y = np.asarray(y, dtype=np.float64)
    shp = y.shape
    H = rht.sylvester(GROUP)
    s = rht.signs(sign_mask).astype(np.float64)
    b = y.reshape(shp[:-1] + (shp[-1] // GROUP, GROUP))
    return ((b @ H.T) / math.sqrt(GROUP) * s).reshape(shp)


def unmask_inverse_rht(c: np.ndarray, mask: np.ndarray, sign_mask: int) -> np.ndarray:
    """H^-1(c o (1 - M)) along rows (float64)."""
    c = np.asarray(c, dtype=np.float64)
    keep = ~unpack_mask(mask, c.shape[1])
    return inverse_rht64(np.where(keep, c, 0.0), sign_mask)


# ---------------------------------------------------------------------------
# The linear layer
# ---------------------------------------------------------------------------

def linear_fwd(x: np.ndarray, w: np.ndarray, seed: int, clip: float):
    """Y = X_q W_q^T with QuEST operands (RHT along K, mask of GEMM 0);
    returns (Y float64, ctx)."""
    g0 = rng.sign_mask(seed, 0)
    xc, xs, xm = quest_quantize(x, g0, clip)
    wc, ws, wm = quest_quantize(w, g0, clip)
    y = mx.gemm(xc, xs, wc, ws)
    return y, {"xq": (xc, xs), "wq": (wc, ws), "mx": xm, "mw": wm, "seed": seed}


def linear_bwd(dy: np.ndarray, ctx: dict):
    """dX = 16/9 H^-1(Q(dY) Q(W_q^T)^T o (1 - M_x)), dW = 16/9 H^-1(Q(dY^T)
    Q(X_q^T)^T o (1 - M_w)), float64."""
    seed = ctx["seed"]
    g0, g1, g2 = (rng.sign_mask(seed, i) for i in range(3))
    dyq = mx.quantize(dy, rounding=mx.SR, axis=mx.ROW, sign_mask=g1, seed=seed, stream=1)
    dyt = mx.quantize(dy, rounding=mx.SR, axis=mx.COL, sign_mask=g2, seed=seed, stream=3)
    wt = requantize(*ctx["wq"], g1, seed, 2)
    xt = requantize(*ctx["xq"], g2, seed, 4)
    dx = unmask_inverse_rht(mx.gemm(*dyq, *wt, alpha=mx.ALPHA_BWD), ctx["mx"], g0)
    dw = unmask_inverse_rht(mx.gemm(*dyt, *xt, alpha=mx.ALPHA_BWD), ctx["mw"], g0)
    return dx, dw


def expected_grads(dy: np.ndarray, ctx: dict):
    """E[dX], E[dW] over the backward's random draws: the SR operands are
    unbiased and the backward RHT cancels in each product, so
    E[dX] = H^-1((dY deq(W_q)) o (1 - M_x)), E[dW] = H^-1((dY^T deq(X_q)) o (1 - M_w))."""
    g0 = rng.sign_mask(ctx["seed"], 0)
    d = np.asarray(dy, dtype=np.float64)
    wq = mx.dequantize(*ctx["wq"])
    xq = mx.dequantize(*ctx["xq"])
    return (unmask_inverse_rht(d @ wq, ctx["mx"], g0),
            unmask_inverse_rht(d.T @ xq, ctx["mw"], g0))
