"""A second, independent implementation of the MXFP4 GEMM as a cross-check:
hipBLASLt's block-scaled FP4 GEMM (E2M1 operands, one E8M0 scale per 32
elements along K, fp32 accumulation; reached through libfp4mx_vendor.so)
against fp4mx_gemm on the same random operands, every output element.

Each of the two is within the fp32 accumulation bound u (K/16 + 8) |alpha| S
of the exact product (S = |A| |B|^T, from the oracle's dequantization), so
they differ by at most twice that.  Every heuristic algorithm hipBLASLt
offers for the shape is compared.  Skipped when the hipBLASLt in the process
offers no MXFP4 algorithm for the shape."""
import ctypes as C

import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd.binding import _stream
from oracle import mx

from gpu_util import assert_gemm_close, cpu, gemm_bound_factor, log, vendor_lib

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)  # hipBLASLt's first handle can take minutes to create
@pytest.mark.parametrize("m,n,k", [(1024, 1536, 2048), (2048, 1024, 4096)])
def test_vendor_gemm_matches(m, n, k):
    log("vendor gemm %dx%dx%d" % (m, n, k))
    V = vendor_lib()
    plan, nalg = C.c_void_p(), C.c_int()
    st = V.fp4mx_vendor_plan_create(m, n, k, C.byref(plan), C.byref(nalg))
    if st != 0:
        pytest.skip("hipBLASLt offers no MXFP4 algorithm for %dx%dx%d (status %d)" % (m, n, k, st))
    try:
        g = torch.Generator(device="cuda").manual_seed(m + n + k)

        def padded(rows, cols, lo, hi):
            # operands sit at the start of buffers 1 MiB longer than they are
            t = torch.randint(lo, hi, (rows * cols + (1 << 20),), dtype=torch.uint8, device="cuda", generator=g)
            return t[:rows * cols].view(rows, cols)
        a, as_ = padded(m, k // 2, 0, 256), padded(m, k // 32, 118, 131)
        b, bs = padded(n, k // 2, 0, 256), padded(n, k // 32, 118, 131)
        alpha = 1.5
        ours = fq.gemm(fq.MXTensor(a, as_), fq.MXTensor(b, bs), alpha=alpha)
        a64 = mx.dequantize(cpu(a), cpu(as_))
        b64 = mx.dequantize(cpu(b), cpu(bs))
        assert_gemm_close(cpu(ours), a64, b64, alpha, "fp4mx_gemm %dx%dx%d" % (m, n, k))
        S = abs(alpha) * (np.abs(a64) @ np.abs(b64).T)
        bound = 2.0 * gemm_bound_factor(k) * S
        o = cpu(ours).astype(np.float64)
        for al in range(nalg.value):
            c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
            st = V.fp4mx_vendor_gemm(plan, al, a.data_ptr(), as_.data_ptr(), b.data_ptr(), bs.data_ptr(),
                                     alpha, c.data_ptr(), _stream(c.device))
            assert st == 0, ("hipBLASLt call failed", al, st)
            torch.cuda.synchronize()
            v = cpu(c).astype(np.float64)
            err = np.abs(v - o)
            ratio = float(np.max(err / np.where(bound > 0, bound, 1.0)))
            log("  algorithm %d: max |vendor - ours| / (2 x bound) %.3f" % (al, ratio))
            assert np.isfinite(v).all(), ("non-finite vendor output", al)
            assert (err <= bound).all(), ("hipBLASLt and fp4mx_gemm differ beyond twice the bound", al, ratio)
    finally:
        V.fp4mx_vendor_plan_destroy(plan)
