"""fp4nv_msedn_quantize_noalloc (MS-EDEN with the library's static scratch)
against fp4nv_msedn_quantize (caller workspace), through the C ABI: identical
codes, E4M3 scales, tensor scale and EDEN factors, on consecutive calls of
decreasing size (the second call reuses the scratch the first one filled)."""
import numpy as np
import pytest
import torch

import fp4_microscaled_quantized_amd as fq
from fp4_microscaled_quantized_amd import synth
from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream

from gpu_util import assert_bytes_equal, cpu, dev_bf16, log

pytestmark = pytest.mark.gpu


def _outputs(orow, ocol):
    dev = "cuda"
    return (torch.empty((orow, ocol // 2), dtype=torch.uint8, device=dev),
            torch.empty((orow, ocol // 16), dtype=torch.uint8, device=dev),
            torch.empty(1, dtype=torch.float32, device=dev),
            torch.empty((orow, ocol // 128), dtype=torch.float32, device=dev))


def _compare(rows, cols, axis, seed):
    L = fq.lib()
    log("no-alloc MS-EDEN", rows, cols, "axis", axis, "seed", seed)
    x = dev_bf16(synth.normal_with_outliers((rows, cols), seed, 2))
    orow, ocol = (rows, cols) if axis == fq.ROW else (cols, rows)
    a, b = _outputs(orow, ocol), _outputs(orow, ocol)
    ws = torch.empty(L.fp4nv_msedn_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    _check(L.fp4nv_msedn_quantize(_ptr(x), rows, cols, cols, axis, 6.0, seed, 1, 5, _ptr(a[0]), _ptr(a[1]),
                                  _ptr(a[2]), _ptr(a[3]), _ptr(ws), ws.numel(), _stream()))
    _check(L.fp4nv_msedn_quantize_noalloc(_ptr(x), rows, cols, cols, axis, 6.0, seed, 1, 5, _ptr(b[0]),
                                          _ptr(b[1]), _ptr(b[2]), _ptr(b[3]), _stream()))
    torch.cuda.synchronize()
    bits = lambda t: cpu(t).view(np.uint32)
    assert_bytes_equal(cpu(b[0]), cpu(a[0]), "codes")
    assert_bytes_equal(cpu(b[1]), cpu(a[1]), "E4M3 scales")
    assert_bytes_equal(bits(b[2]), bits(a[2]), "tensor scale")
    assert_bytes_equal(bits(b[3]), bits(a[3]), "EDEN factors")


@pytest.mark.parametrize("axis,sizes", [
    (fq.ROW, [(16384, 8192), (384, 640)]),     # the largest input the scratch holds, then a small one
    (fq.COL, [(4096, 2048), (256, 384)]),
])
def test_noalloc_matches_workspace_form(axis, sizes):
    for i, (rows, cols) in enumerate(sizes):
        _compare(rows, cols, axis, seed=11 + i)
