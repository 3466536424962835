"""Shared helpers for the GPU parity tests (inputs from the seeded generators,
device transfer, comparisons).  No quantization arithmetic lives here."""
import sys

import numpy as np
import torch

from fp4_microscaled_quantized_amd import synth


def log(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bits -> CUDA bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_f32(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits)


def cpu(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def rel_fro(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError("%s: %d of %d bytes differ; first at %s: got %s want %s"
                             % (what, bad[0].size, got.size, i, got[i], want[i]))


def edge_case_tensor(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """bf16 bits with the quantizer's corner cases planted in separate 32-blocks."""
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((rows, cols)).astype(np.float32)
    blocks = [
        np.zeros(32),                                       # all-zero group
        -np.zeros(32),                                      # negative zeros
        np.full(32, 1e-39),                                 # bf16 subnormals
        rs.standard_normal(32) * 1e-38,                     # tiny: scale code 0
        rs.standard_normal(32) * 1e37,                      # huge
        np.full(32, 3.0e38),                                # sums overflow in the transform
        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4),   # E2M1 ties (x4 scale)
        np.where(np.arange(32) == 5, np.nan, 1.0),          # NaN
        np.where(np.arange(32) == 9, np.inf, 1.0),          # +Inf
        np.where(np.arange(32) == 0, -np.inf, 0.5),         # -Inf
        np.ldexp(1.0, np.arange(32) - 16),                  # wide dynamic range
        np.full(32, 6.0), np.full(32, 8.0), np.full(32, 7.99),
    ]
    flat = x.reshape(-1, 32)
    for i, b in enumerate(blocks):
        if i * 7 < flat.shape[0]:
            flat[i * 7] = np.asarray(b, dtype=np.float32)
    return synth.f32_to_bf16_bits(flat.reshape(rows, cols))


# ---------------------------------------------------------------------------
# Element-wise GEMM check.
#
# The FP4 GEMM multiplies E2M1 values scaled by powers of two (each product is
# exact) and accumulates in fp32: every MFMA adds a 64-element K slice to the
# fp32 accumulator.  Modelling each MFMA as at most two fp32 roundings of a
# partial sum bounded by S = sum_k |a_ik b_jk|, plus one rounding for alpha and
# one for alpha's own fp32 value, gives
#     |C_gpu - alpha C_64| <= u (K/32 + 4) |alpha| S,   u = 2^-24.
# The check uses twice that, u (K/16 + 8) |alpha| S, so every output element
# is held to a few fp32 ulps of its own magnitude scale; a wrong group scale,
# a misplaced tile or a dropped K slice moves elements by far more.
# ---------------------------------------------------------------------------

def gemm_bound_factor(k: int) -> float:
    return 2.0 ** -24 * (k / 16 + 8)


def assert_gemm_close(got, a64, b64, alpha, what, tol=1e-5, extra_bound=None):
    """got [M,N] (fp32 from the GPU) against alpha * a64 @ b64^T in fp64:
    element-wise within the accumulation bound (plus ``extra_bound`` [M,N] if
    given) and within ``tol`` relative Frobenius.  Non-finite expected entries
    must match (NaN for NaN)."""
    got = np.asarray(got, dtype=np.float64)
    want = alpha * (a64 @ b64.T)
    S = abs(alpha) * (np.abs(a64) @ np.abs(b64).T)
    bound = gemm_bound_factor(a64.shape[1]) * S
    if extra_bound is not None:
        bound = bound + extra_bound
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got[~fin]), np.isnan(want[~fin])), what + ": non-finite entries differ"
    err = np.abs(got[fin] - want[fin])
    b = bound[fin]
    bad = err > b
    ratio = float(np.max(err / np.where(b > 0, b, 1.0))) if err.size else 0.0
    fro = rel_fro(got[fin], want[fin])
    log("  %s: max err/bound %.3f, rel fro %.2e, %d elements" % (what, ratio, fro, err.size))
    if bad.any():
        i = np.argmax(bad)
        raise AssertionError("%s: %d of %d elements beyond the bound; first at flat %d: got %r want %r "
                             "bound %r" % (what, int(bad.sum()), bad.size, i, got[fin][i], want[fin][i], b[i]))
    assert fro <= tol, (what, fro)


def edge_case_tensor_cols(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """edge_case_tensor with its special 32-blocks running down columns: the
    column-axis quantizer sees them as whole groups."""
    return np.ascontiguousarray(edge_case_tensor(cols, rows, seed).T)


# ---------------------------------------------------------------------------
# hipBLASLt's MXFP4 GEMM (libfp4mx_vendor.so, built beside libfp4mx.so).
# ---------------------------------------------------------------------------
_vendor = None


def vendor_lib():
    """ctypes handle of libfp4mx_vendor.so with its three entry points typed."""
    import ctypes as C
    import os
    global _vendor
    if _vendor is None:
        from fp4_microscaled_quantized_amd import binding
        path = os.path.join(os.path.dirname(binding.LIB_PATH), "libfp4mx_vendor.so")
        L = C.CDLL(path)
        L.fp4mx_vendor_plan_create.restype = C.c_int
        L.fp4mx_vendor_plan_create.argtypes = [C.c_int64] * 3 + [C.POINTER(C.c_void_p), C.POINTER(C.c_int)]
        L.fp4mx_vendor_gemm.restype = C.c_int
        L.fp4mx_vendor_gemm.argtypes = ([C.c_void_p, C.c_int] + [C.c_void_p] * 4
                                        + [C.c_float, C.c_void_p, C.c_void_p])
        L.fp4mx_vendor_plan_destroy.restype = None
        L.fp4mx_vendor_plan_destroy.argtypes = [C.c_void_p]
        _vendor = L
    return _vendor
