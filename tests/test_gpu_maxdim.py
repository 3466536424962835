"""GPU parity at the largest accepted sizes (FP4MX_MAX_DIM = 2^21): the
quantizers on a 32 x 2^21 matrix (checked against the oracle on column
slices, the last one included), the GEMM with K = 2^21, and GEMM outputs with
ldc = 2^21, where each 256-row tile's output range reaches the 2^31-byte limit
(no store may land outside [:, :n])."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from oracle import mx, nvfp4, quest, rng

from gpu_util import assert_bytes_equal, cpu, dev_bf16, host_f32, log, rel_fro

pytestmark = pytest.mark.gpu

MAXD = 1 << 21
SLICES = [0, 700 * 1024, MAXD - 2048]   # column offsets (multiples of 128), the last at the edge
W = 2048


@pytest.fixture(scope="module")
def wide():
    bits = synth.normal_with_outliers((32, MAXD), 21, 0)
    return bits, dev_bf16(bits)


def test_mx_quantize_max_cols(wide):
    bits, x = wide
    m1, m2 = rng.sign_mask(21, 1), rng.sign_mask(21, 2)
    log("max cols: mx row RTN + col SR", x.shape)
    ro = fq.hadamard_quantize(x, axis=fq.ROW, rounding=fq.RTN, mask=m1)
    co = fq.hadamard_quantize(x, axis=fq.COL, rounding=fq.SR, mask=m2, seed=8, rng_stream=4)
    torch.cuda.synchronize()
    rc, rs, cc, cs = cpu(ro.codes), cpu(ro.scales), cpu(co.codes), cpu(co.scales)
    for c0 in SLICES:
        xs = host_f32(bits[:, c0:c0 + W])
        wc, ws = mx.quantize(xs, rounding=mx.RTN, axis=mx.ROW, sign_mask=m1)
        assert_bytes_equal(rc[:, c0 // 2:(c0 + W) // 2], wc, "row codes @%d" % c0)
        assert_bytes_equal(rs[:, c0 // 32:(c0 + W) // 32], ws, "row scales @%d" % c0)
        wc, ws = mx.quantize(xs, rounding=mx.SR, axis=mx.COL, sign_mask=m2, seed=8, stream=4,
                             row_ids=np.arange(c0, c0 + W))
        assert_bytes_equal(cc[c0:c0 + W], wc, "col codes @%d" % c0)
        assert_bytes_equal(cs[c0:c0 + W], ws, "col scales @%d" % c0)


def test_quest_and_nvfp4_max_cols(wide):
    bits, x = wide
    m = rng.sign_mask(21, 3)
    log("max cols: quest, nvfp4 4/6", x.shape)
    qo, qm = fq.quest_quantize(x, mask=m)
    nv = fq.nv_quantize46(x)
    torch.cuda.synchronize()
    qc, qs, qmk = cpu(qo.codes), cpu(qo.scales), cpu(qm)
    nc, ns, g = cpu(nv.codes), cpu(nv.scales), cpu(nv.tensor_scale)[0]
    assert g == nvfp4.tensor_scale(host_f32(bits))
    for c0 in SLICES:
        xs = host_f32(bits[:, c0:c0 + W])
        wc, ws, wm = quest.quest_quantize(xs, m, fq.QUEST_CLIP)
        assert_bytes_equal(qc[:, c0 // 2:(c0 + W) // 2], wc, "quest codes @%d" % c0)
        assert_bytes_equal(qs[:, c0 // 32:(c0 + W) // 32], ws, "quest scales @%d" % c0)
        assert_bytes_equal(qmk[:, c0 // 8:(c0 + W) // 8], wm, "quest mask @%d" % c0)
        wc, ws, _ = nvfp4.quantize46(xs, True, g=np.float32(g))
        assert_bytes_equal(nc[:, c0 // 2:(c0 + W) // 2], wc, "nv codes @%d" % c0)
        assert_bytes_equal(ns[:, c0 // 16:(c0 + W) // 16], ws, "nv scales @%d" % c0)


def test_gemm_max_k():
    """K = 2^21 on one 32 x 32 tile, operands drawn directly as seeded random
    E2M1 codes and E8M0 scales 2^-9..2^2.  fp32 accumulation over K terms: the
    tolerance is 4 sqrt(K) 2^-24 (rounding errors of random sign)."""
    k = MAXD
    log("gemm max K", k)
    g = np.random.default_rng(24)
    a = (g.integers(0, 256, (32, k // 2), dtype=np.uint8), g.integers(118, 130, (32, k // 32), dtype=np.uint8))
    b = (g.integers(0, 256, (32, k // 2), dtype=np.uint8), g.integers(118, 130, (32, k // 32), dtype=np.uint8))
    A = fq.MXTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda())
    B = fq.MXTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda())
    c = fq.gemm(A, B)
    torch.cuda.synchronize()
    err = rel_fro(cpu(c), mx.gemm(*a, *b))
    log("  rel err %.2e" % err)
    assert err <= 4 * np.sqrt(k) * 2.0 ** -24


@pytest.mark.parametrize("kind", ["f32", "bf16", "irht"])
def test_gemm_max_ldc(kind):
    """256 x 96 output written into a 256 x 2^21 buffer: values equal the
    oracle's, and every element outside [:, :96] keeps its sentinel."""
    m, n, k, ldc = 256, 96, 128, MAXD
    log("gemm max ldc", kind)
    a = mx.quantize(host_f32(synth.normal((m, k), 1.0, 23, 0)), rounding=mx.SR, sign_mask=7, seed=1, stream=1)
    b = mx.quantize(host_f32(synth.normal((n, k), 1.0, 23, 1)), rounding=mx.SR, sign_mask=7, seed=1, stream=2)
    A = fq.MXTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda())
    B = fq.MXTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda())
    want = mx.gemm(*a, *b, alpha=mx.ALPHA_BWD)
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    c = torch.full((m, ldc), 5.0, dtype=dt, device="cuda")
    if kind == "f32":
        fq.gemm(A, B, alpha=16 / 9, out=c[:, :n])
    elif kind == "bf16":
        fq.gemm_bf16(A, B, alpha=16 / 9, out=c[:, :n])
    else:
        bm = np.random.default_rng(4).random((m, n)) < 0.05
        mk = np.packbits(bm, axis=1, bitorder="little")
        sm = rng.sign_mask(23, 0)
        fq.gemm_unmask_irht(A, B, torch.from_numpy(mk).cuda(), alpha=16 / 9, mask=sm, out=c[:, :n])
        want = quest.unmask_inverse_rht(want, mk, sm)
    torch.cuda.synchronize()
    outside = int((c[:, n:] != 5.0).sum().item())
    assert outside == 0
    got = cpu(c[:, :n].float())
    assert rel_fro(got, want) <= (2.0 ** -8 if kind == "bf16" else 1e-5)
    del c
    torch.cuda.empty_cache()
