"""Block-32 randomized Hadamard transform (RHT) along a tensor's last axis.

Test infrastructure (see the package docstring).

Sources:
* "Quartet: Native FP4 Training Can Be Optimal for Large Language Models",
  section "The Hadamard Transform: Why It Is Necessary and How It Is
  Implemented": blocks of g = 32 along the feature (GEMM inner) dimension,
  the Sylvester/Kronecker recursion, normalisation 1/sqrt(g) making the
  transform orthogonal, random sign flips for the randomized variant, and the
  cost "O(g log g) = 5 operations per element" of the fast Walsh-Hadamard
  transform; "The GPU Kernel Implementation", Stage 1: the transform produces
  FP32 output.
* "Quartet II ...", section "MS-EDEN", Step 1: RHT = Hadamard times random
  diagonal sign flips, one sign pattern shared by every block of a tensor.
* "Bridging the Gap ...", "Block-Wise Hadamard Rotation (Ingredient 3)":
  H_k H_k^T = k I, so rotating both operands along the inner dimension leaves
  the product unchanged.

Readings taken (the pages are loose here):
* The unnormalised +-1 Sylvester matrix H[i][j] = (-1)^popcount(i & j) is
  applied and one overall factor c = fl32(1/sqrt(32)) follows; the printed
  recursion normalises twice and is not taken literally.
* One random diagonal D (bit j of ``sign_mask`` set <=> s_j = -1) is applied
  before H; a second flip after H would cancel in A B^T exactly as this one
  does.
* The fp32 evaluation order is the FWHT: radix-2 butterflies
  (a, b) -> (fl(a+b), fl(a-b)) on index pairs (i, i+h), i & h == 0, for
  h = 1, 2, 4, 8, 16 in that order, then y_i = fl(t_i * c).
"""
from __future__ import annotations

import numpy as np

G = 32
INV_SQRT_G = np.float32(1.0 / np.sqrt(32.0))          # 0x3E3504F3


def signs(sign_mask: int) -> np.ndarray:
    """+-1 vector (float32) from the 32-bit mask."""
    return np.array([-1.0 if (sign_mask >> j) & 1 else 1.0 for j in range(G)],
                    dtype=np.float32)


def fwht32(t: np.ndarray) -> np.ndarray:
    """Unnormalised FWHT over the last axis (length 32), float32 butterflies."""
    t = np.array(t, dtype=np.float32, copy=True)
    h = 1
    while h < G:
        for i in range(G):
            if i & h:
                continue
            a = t[..., i].copy()
            b = t[..., i + h].copy()
            t[..., i] = a + b
            t[..., i + h] = a - b
        h *= 2
    return t


def rht32(x: np.ndarray, sign_mask: int) -> np.ndarray:
    """y = c * H (s * x) per 32-block of the last axis, all in float32."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    assert shp[-1] % G == 0
    blocks = x.reshape(shp[:-1] + (shp[-1] // G, G))
    t = fwht32(blocks * signs(sign_mask))
    y = t * INV_SQRT_G
    return y.reshape(shp)


def sylvester(n: int) -> np.ndarray:
    """The +-1 Sylvester-ordered Hadamard matrix of order n (n a power of 2)."""
    idx = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(idx[:, None] & idx[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)
