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
