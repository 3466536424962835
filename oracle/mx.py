"""MXFP4 quantizers, dequantization, the FP4 GEMM and the linear layer.

Test infrastructure (see the package docstring).

MXFP4 operand layout (both the oracle's outputs and the library's):
codes  uint8 [rows, cols/2]: element 2j in the low nibble of byte j, 2j+1 in
       the high nibble; every group of 32 consecutive elements along a row
       shares one scale;
scales uint8 [rows, cols/32]: E8M0 bytes.

Sources:
* "Quartet: Native FP4 Training ...": "The QuEST Forward-Pass Quantization"
  (groups of 32 along the GEMM K dimension, M x ceil(K/32) scales), "The 3/4
  rescaling factor" (SR(3/4 G_h), 16/9 after the GEMM), "The GPU Kernel
  Implementation" (Stage 1 group max -> E8M0, Stage 2 D = C + (A SFA)(B SFB)
  with FP32 accumulation), "The Complete Quartet Algorithm" (forward and
  backward GEMMs, shared seed for a GEMM's two operands, saved context).
* "Quartet II ...": "The Complete Quartet II Computation Graph" (RHT along the
  inner dimension of every GEMM on both operands with the same seed, no
  inverse transform) and "Big-Picture Architecture".
"""
from __future__ import annotations

import numpy as np

from . import formats, rht, rng

RTN, SR = 0, 1
ROW, COL = 0, 1
ALPHA_BWD = 16.0 / 9.0


def _scale_inv(code: np.ndarray) -> np.ndarray:
    """2^(127 - code) as float32 (exactly representable for code <= 254)."""
    return np.ldexp(np.float32(1.0), 127 - code.astype(np.int32)).astype(np.float32)


def quantize(x: np.ndarray, *, rounding: int, axis: int = ROW, hadamard: bool = True,
             sign_mask: int = 0, seed: int = 0, stream: int = 0, row_ids=None):
    """MXFP4-quantize one GEMM operand.

    x        float32 [R, C] holding bfloat16 values.
    axis     ROW: groups of 32 along each row; output codes [R, C/2].
             COL: the operand is x^T (groups along columns of x);
             output codes [C, R/2] (the transposed operand, K-major).
    rounding RTN (forward): v = fl(y * 2^(127-e)), E2M1 round-to-nearest-even,
             saturating.  SR (backward): v = fl(y * (3/4 * 2^(127-e))) and
             stochastic rounding (``formats.e2m1_sr_carry``: up iff
             floor(p * 2^22) + (r >> 10) >= 2^22); |v| < 6 always holds,
             so nothing clips.
    hadamard apply the block-32 RHT with ``sign_mask`` first.

    The scale byte e comes from the group maximum of y (before the 3/4), see
    ``formats.e8m0_code``.  Reading: the pages say the backward scale is
    "determined by the 3/4 rescaling"; taking the scale from the unscaled
    maximum and scaling the elements by 3/4 is the reading under which the
    prescale makes SR clip-free, which is its stated purpose.
    A group holding a non-finite value (after the transform) gets scale 0xFF
    and all-zero element codes.
    The SR draw for output element (r, c) uses index r * cols_out + c.
    ``row_ids`` (optional) gives the output rows' indices in the full operand
    when only some of its rows are passed (sampled checks); the rows are
    independent, so this is the same computation restricted to those rows.
    """
    a = np.asarray(x, dtype=np.float32)
    if axis == COL:
        a = np.ascontiguousarray(a.T)
    R, C = a.shape
    if C % 32:
        raise ValueError("the grouped dimension must be a multiple of 32")
    y = rht.rht32(a, sign_mask) if hadamard else a.copy()
    blocks = y.reshape(R, C // 32, 32)
    with np.errstate(invalid="ignore", over="ignore"):
        finite = np.all(np.isfinite(blocks), axis=2)
        amax = np.where(finite, np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0)), axis=2), 0)
    code = formats.e8m0_code(amax.astype(np.float32))
    inv = _scale_inv(code)[:, :, None]
    if rounding == RTN:
        v = (blocks * inv).astype(np.float32)
        q = formats.e2m1_rtn(v)
    elif rounding == SR:
        f = (np.float32(0.75) * inv).astype(np.float32)      # exact: 3 * 2^(125-e)
        v = (blocks * f).astype(np.float32)
        rid = np.arange(R, dtype=np.uint64) if row_ids is None else np.asarray(row_ids, dtype=np.uint64)
        idx = (rid[:, None] * np.uint64(C)
               + np.arange(C, dtype=np.uint64)[None, :]).reshape(R, C // 32, 32)
        r = rng.bits(seed, stream, idx)
        v = np.where(finite[:, :, None], v, 0).astype(np.float32)
        q = formats.e2m1_sr_carry(v, r)
    else:
        raise ValueError("rounding must be RTN or SR")
    q = np.where(finite[:, :, None], q, 0).astype(np.uint8)
    code = np.where(finite, code, 255).astype(np.uint8)
    q = q.reshape(R, C)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, code


def unpack(codes: np.ndarray) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] 4-bit codes."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 operand -> float64 values q * 2^(e-127)."""
    q = formats.e2m1_decode(unpack(codes))
    s = formats.e8m0_value(scales)
    return q * np.repeat(s, 32, axis=1)


def gemm(a_codes, a_scales, b_codes, b_scales, alpha: float = 1.0) -> np.ndarray:
    """C = alpha * deq(A) deq(B)^T in float64 (A [M,K], B [N,K], both K-major).

    Plain definition of Stage 2 (D = (A x SFA)(B x SFB)); every product of an
    E2M1 value and a power of two is exact in float64.
    """
    A = dequantize(a_codes, a_scales)
    B = dequantize(b_codes, b_scales)
    return alpha * (A @ B.T)


def linear_fwd(x: np.ndarray, w: np.ndarray, seed: int, want_ctx: bool = True):
    """Forward of the fully-FP4 linear layer Y = X W^T.

    X [M,K], W [N,K] float32 holding bfloat16 values.  Both operands get the
    RHT along K with the GEMM-0 sign mask and RTN quantization; Y is the fp32
    product (returned here in float64).  The saved context holds the backward
    operands made from the same X and W: X^T and W^T quantized along M and N
    with SR (RHT masks of GEMMs 2 and 1, RNG streams 4 and 2).
    """
    g0, g1, g2 = (rng.sign_mask(seed, i) for i in range(3))
    xq = quantize(x, rounding=RTN, axis=ROW, sign_mask=g0)
    wq = quantize(w, rounding=RTN, axis=ROW, sign_mask=g0)
    y = gemm(*xq, *wq)
    if not want_ctx:
        return y, None
    ctx = {
        "xt": quantize(x, rounding=SR, axis=COL, sign_mask=g2, seed=seed, stream=4),
        "wt": quantize(w, rounding=SR, axis=COL, sign_mask=g1, seed=seed, stream=2),
        "seed": seed,
    }
    return y, ctx


def linear_bwd(dy: np.ndarray, ctx: dict):
    """Backward: dX = 16/9 * Q(dY) Q(W^T)^T along N, dW = 16/9 * Q(dY^T) Q(X^T)^T along M.

    dY [M,N] float32 holding bfloat16 values; both dY operands are SR-quantized
    (streams 1 and 3) with the RHT of their GEMM.
    """
    seed = ctx["seed"]
    g1, g2 = rng.sign_mask(seed, 1), rng.sign_mask(seed, 2)
    dyq = quantize(dy, rounding=SR, axis=ROW, sign_mask=g1, seed=seed, stream=1)
    dyt = quantize(dy, rounding=SR, axis=COL, sign_mask=g2, seed=seed, stream=3)
    dx = gemm(*dyq, *ctx["wt"], alpha=ALPHA_BWD)
    dw = gemm(*dyt, *ctx["xt"], alpha=ALPHA_BWD)
    return dx, dw
