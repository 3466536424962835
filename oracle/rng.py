"""Counter-based random bits for stochastic rounding and the RHT sign masks.

Test infrastructure (see the package docstring).

The pages only fix that the randomness is seeded and that the seed is passed
explicitly ("Quartet: Native FP4 Training ...", section "The Hadamard
Transform ...", randomized Hadamard on the backward pass; "Quartet II ...",
"The Complete Quartet II Computation Graph", step 3: the same seed for both
operands of a GEMM).  Reading taken here: one counter-based generator built
from two published mixing functions,

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; Vigna's reference ``splitmix64.c``): the output
  for state s is mix64(s + 0x9E3779B97F4A7C15);
* the MurmurHash3 32-bit finalizer ``fmix32`` (Appleby, SMHasher).

Per (seed, stream): key = splitmix64(seed XOR (stream << 32)).
Per element with output-operand linear index i = row * cols + col:
    r(i) = fmix32(lo32(i) ^ lo32(key) ^ fmix32(hi32(i) ^ hi32(key))).
The E2M1 stochastic roundings (the MXFP4 quantizers and the NVFP4 SR
baseline) draw u = (r >> 10) * 2^-22 (formats.e2m1_sr_carry); MS-EDEN's E4M3
scale rounding draws u = (r >> 8) * 2^-24.
RHT sign mask of GEMM g: lo32(splitmix64(seed XOR ((0x5100 + g) << 32))).
"""
from __future__ import annotations

import numpy as np

M64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(x: int) -> int:
    """SplitMix64 output for state ``x`` (the state is advanced by the golden
    gamma first, then mixed with the variant-13 finalizer)."""
    z = (x + GOLDEN_GAMMA) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def fmix32(h):
    """MurmurHash3 32-bit finalizer; works on Python ints and uint32 arrays."""
    if isinstance(h, np.ndarray):
        h = h.astype(np.uint32)
        h = h ^ (h >> np.uint32(16))
        h = (h.astype(np.uint64) * 0x85EBCA6B).astype(np.uint32)
        h = h ^ (h >> np.uint32(13))
        h = (h.astype(np.uint64) * 0xC2B2AE35).astype(np.uint32)
        return h ^ (h >> np.uint32(16))
    h &= 0xFFFFFFFF
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & 0xFFFFFFFF
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & 0xFFFFFFFF
    return h ^ (h >> 16)


def stream_key(seed: int, stream: int) -> int:
    return splitmix64((seed ^ (stream << 32)) & M64)


def bits(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """32 random bits for each 64-bit element index in ``idx``."""
    k = stream_key(seed, stream)
    idx = np.asarray(idx, dtype=np.uint64)
    lo = (idx & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (idx >> np.uint64(32)).astype(np.uint32)
    inner = fmix32(hi ^ np.uint32(k >> 32))
    return fmix32(lo ^ np.uint32(k & 0xFFFFFFFF) ^ inner)


def uniform24(r: np.ndarray) -> np.ndarray:
    """u = (r >> 8) * 2^-24 in [0, 1), as float64 (exact)."""
    return (np.asarray(r, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) * 2.0 ** -24


def sign_mask(seed: int, gemm_id: int) -> int:
    """32-bit RHT sign mask shared by both operands of GEMM ``gemm_id``
    (0 = forward, 1 = input gradient, 2 = weight gradient)."""
    return splitmix64((seed ^ ((0x5100 + gemm_id) << 32)) & M64) & 0xFFFFFFFF
