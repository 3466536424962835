"""CPU oracle for the fully-FP4 (MXFP4 / NVFP4) quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; both are fed the same seeded inputs.

It is a plain, slow, written-out restatement of what the pages compute:

* "Quartet: Native FP4 Training Can Be Optimal for Large Language Models"
  (the block Hadamard transform, MXFP4 quantization with RTN forward / SR
  backward and the 3/4 and 16/9 rescales, the three FP4 GEMMs);
* "Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased
  Gradient Estimation" (the NVFP4 format, Four-over-Six, inner-dimension RHT);
* "Bridging the Gap Between Promise and Performance for Microscaling FP4
  Quantization" (the E2M1 / E8M0 / E4M3 formats, block Hadamard rotation).

Every function names the passage it follows.  Where the pages leave a step
open the reading taken is stated in the function's docstring.

Pinned: codecs (exhaustive / library routes), the FWHT (Sylvester matrix,
orthogonality), the RNG (published test vectors), SR (exact probabilities,
unbiasedness), GEMM (brute-force triple loop), linear backward (expectation
equals the exact gradient), NVFP4 RTN and RTN+4/6 (the pages' Table 1 MSEs),
MS-EDEN and the NVFP4 SR baseline (Table 1 MSEs, the EDEN correction range,
RHT_128 structure, unbiasedness of the scale rounding and of the product),
QuEST (the Gaussian objective against quadrature and Monte Carlo, its
minimum, sigma and thresholds against fp64, reduction of clipping groups to MX
RTN, the page's MSE ranking QuEST < RTN < SR, power-of-two invariance) and the
Quartet backward in the rotated basis (inverse RHT against the matrix
inverse, mask correction, re-quantization and the whole backward unbiased),
and the Quartet II graph with re-quantized saved NVFP4 operands (de-quantization
as the rounded exact product, Table 1's MS-EDEN error on re-quantized
operands, unbiased backward).
The FP8 staging of the NVFP4 GEMM is a design of this library that the pages
do not describe; it is pinned exhaustively (every E2M1 code under every pair of
positive finite E4M3 group scales of a 32-block) against an independent route:
a brute-force block exponent, the exact product and torch's float8_e4m3fn
rounding.
"""

from . import formats, rng, rht, mx, nvfp4, msedn, quest, quartet2  # noqa: F401
