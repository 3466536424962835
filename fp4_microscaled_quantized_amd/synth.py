"""Seeded synthetic inputs for the fully-FP4 linear layer workloads.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the quantizer, transform or GEMM arithmetic.  Both the CPU oracle and
the GPU path are fed from the buffers made here, so they see identical bits.

Recipe: ``numpy.random.default_rng([seed, tensor_id])`` draws in float64,
the draw is rounded to float32 and then to bfloat16 with round-to-nearest-even.
Tensor ids: X = 0, W = 1, dY = 2.

The workloads stand in for the LLM layer activations, weights and gradients the
pages train on (Llama-family linear layers, C4 / FineWeb-Edu activations),
which are not available here.
"""
from __future__ import annotations

import numpy as np

TENSOR_X, TENSOR_W, TENSOR_DY = 0, 1, 2


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Non-finite inputs keep their class (NaN stays NaN, Inf stays Inf).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id])


def _to_bf16(x64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x64.astype(np.float32))


def normal(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    """i.i.d. N(0, std^2) as bfloat16 bits."""
    g = _rng(seed, tensor_id)
    return _to_bf16(g.standard_normal(shape) * std)


def normal_with_outliers(shape, seed: int, tensor_id: int, frac: float = 0.01,
                         factor: float = 20.0) -> np.ndarray:
    """N(0,1) with a Bernoulli(frac) subset of entries multiplied by ``factor``."""
    g = _rng(seed, tensor_id)
    x = g.standard_normal(shape)
    m = g.random(shape) < frac
    x[m] *= factor
    return _to_bf16(x)


def normal_with_outlier_channels(shape, seed: int, tensor_id: int, n_channels: int,
                                 factor: float) -> np.ndarray:
    """N(0,1) with ``n_channels`` columns (chosen by a seeded permutation) scaled."""
    g = _rng(seed, tensor_id)
    x = g.standard_normal(shape)
    cols = g.permutation(shape[1])[:n_channels]
    x[:, cols] *= factor
    return _to_bf16(x)


def normal_and_student_t(shape, seed: int, tensor_id: int, nu: float = 3.0) -> np.ndarray:
    """First half of the rows N(0,1), second half Student-t(nu)."""
    g = _rng(seed, tensor_id)
    r = shape[0]
    x = np.empty(shape, dtype=np.float64)
    x[: r // 2] = g.standard_normal((r // 2,) + tuple(shape[1:]))
    x[r // 2:] = g.standard_t(nu, (r - r // 2,) + tuple(shape[1:]))
    return _to_bf16(x)


# ---------------------------------------------------------------------------
# The five workloads.  Each returns a dict of bfloat16-bit arrays.
# ---------------------------------------------------------------------------

def tiny_linear(seed: int = 0):
    """X 64x128 and W 128x128, N(0,1) with 1% of entries x20."""
    return {"x": normal_with_outliers((64, 128), seed, TENSOR_X),
            "w": normal_with_outliers((128, 128), seed, TENSOR_W)}


def quantizer_tensor(seed: int = 0, rows: int = 8192, cols: int = 4096):
    """8192x4096: rows [0, R/2) N(0,1), rows [R/2, R) Student-t(3)."""
    return {"x": normal_and_student_t((rows, cols), seed, TENSOR_X)}


def quartet_linear(seed: int = 0, m: int = 8192, n: int = 4096, k: int = 4096):
    """X [m,k] ~ N(0,1), W [n,k] ~ N(0,0.02), dY [m,n] ~ N(0,1e-3) (standard deviations)."""
    return {"x": normal((m, k), 1.0, seed, TENSOR_X),
            "w": normal((n, k), 0.02, seed, TENSOR_W),
            "dy": normal((m, n), 1e-3, seed, TENSOR_DY)}


def llama_ffn_up(seed: int = 0, m: int = 8192, n: int = 14336, k: int = 4096):
    """Llama-3-8B FFN up-projection: X with round(0.005*k) channels x50."""
    nch = int(round(0.005 * k))
    return {"x": normal_with_outlier_channels((m, k), seed, TENSOR_X, nch, 50.0),
            "w": normal((n, k), 0.02, seed, TENSOR_W),
            "dy": normal((m, n), 1e-3, seed, TENSOR_DY)}


def nvfp4_linear(seed: int = 0, m: int = 16384, n: int = 8192, k: int = 8192):
    """NVFP4 forward: X [m,k] ~ N(0,1), W [n,k] ~ N(0,0.02)."""
    return {"x": normal((m, k), 1.0, seed, TENSOR_X),
            "w": normal((n, k), 0.02, seed, TENSOR_W)}
