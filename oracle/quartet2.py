"""The Quartet II linear layer with re-quantization of the saved forward
operands: forward NVFP4 (RTN + Four-over-Six) keeps Q(X) and Q(W); the
backward dequantizes them, transposes them and re-quantizes them with MS-EDEN
along each backward GEMM's inner dimension.

Test infrastructure (see the package docstring).

Sources ("Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased
Gradient Estimation"):
* "The Complete Quartet II Computation Graph": forward RTN + 4/6 with native
  1x16 scales, the quantized W and X saved; per backward GEMM: de-quantize the
  saved tensors, transpose, one RHT seed shared by both operands on the inner
  dimension, MS-EDEN re-quantization of both operands (E and W^T for the input
  gradient, E^T and X for the weight gradient), NVFP4 GEMM; the outputs need
  no inverse RHT.
* "Forward Pass Design: The Representation-Requantization Trade-Off": native
  scales, so the weights are re-quantized on the backward pass.

Readings taken:
* De-quantization to fp32: fl32(q s16 g), one rounding of the exact product
  (q s16 is exact; NVFP4 values are generally not representable in bf16).
* RHT masks and RNG streams are those of the library's bf16 backward: GEMM 1
  (dX = E W, inner N): E rows stream 5, W^T stream 6; GEMM 2 (dW = E^T X,
  inner M): E^T stream 7, X^T stream 8; clip factor s = 6.
* The NVFP4 GEMM is the library's FP8-staged product (``nvfp4.gemm_fp8_staged``).
"""
from __future__ import annotations

import numpy as np

from . import msedn, nvfp4

CLIP = 6.0


def dequantize32(codes, scales, g) -> np.ndarray:
    """Saved NVFP4 operand -> float32 values fl32(q s16 g)."""
    return nvfp4.dequantize(codes, scales, g).astype(np.float32)


def requantize(codes, scales, g, words, seed: int, stream: int, s: float = CLIP,
               row_ids=None, k: int | None = None):
    """Saved NVFP4 operand A [R, C] -> MS-EDEN of A^T [C, R] (128-chunks along
    R).  ``row_ids`` / ``k`` select output rows with the full tensor's range
    exponent, as in ``msedn.msedn_quantize``.  Returns (codes, scales, g, S)."""
    at = np.ascontiguousarray(dequantize32(codes, scales, g).T)
    if row_ids is not None:
        at = np.ascontiguousarray(at[np.asarray(row_ids)])
    return msedn.msedn_quantize(at, words, seed, stream, s, row_ids=row_ids, k=k)


def requant_range_exponent(codes, scales, g, words, s: float = CLIP) -> int:
    at = np.ascontiguousarray(dequantize32(codes, scales, g).T)
    return msedn.msedn_range_exponent(at, words, s)


def linear_fwd(x: np.ndarray, w: np.ndarray):
    """Y (float64) and ctx = {Q(X), Q(W)} (codes, E4M3 scales, tensor scale)."""
    y, xq, wq = nvfp4.linear_fwd(x, w, use_46=True)
    return y, {"xq": xq, "wq": wq}


def linear_bwd(dy: np.ndarray, ctx: dict, seed: int):
    """dX = gemm(MSEDEN(E), MSEDEN(deq(Q(W))^T)), dW = gemm(MSEDEN(E^T),
    MSEDEN(deq(Q(X))^T)), float64."""
    w1, w2 = msedn.sign_mask128(seed, 1), msedn.sign_mask128(seed, 2)
    a = msedn.msedn_quantize(dy, w1, seed, 5, CLIP)[:3]
    b = requantize(*ctx["wq"], w1, seed, 6)[:3]
    dx = nvfp4.gemm_fp8_staged(*a, *b)
    c = msedn.msedn_quantize(np.ascontiguousarray(np.asarray(dy, np.float32).T), w2, seed, 7, CLIP)[:3]
    d = requantize(*ctx["xq"], w2, seed, 8)[:3]
    dw = nvfp4.gemm_fp8_staged(*c, *d)
    return dx, dw


def expected_grads(dy: np.ndarray, ctx: dict):
    """E[dX] = E deq(Q(W)), E[dW] = E^T deq(Q(X)) (float64): MS-EDEN is unbiased
    and the shared RHT cancels in each product."""
    e = np.asarray(dy, dtype=np.float64)
    return e @ nvfp4.dequantize(*ctx["wq"]), e.T @ nvfp4.dequantize(*ctx["xq"])
