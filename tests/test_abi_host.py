"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching a GPU."""
import ctypes as C
import os
import re

import pytest

from fp4_microscaled_quantized_amd import binding
from oracle import rng

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4mx.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"FP4MX_API\s+[\w\s\*]*?\b(fp4(?:mx|nv)_\w+)\s*\(", txt)))


def test_header_declares_entry_points():
    names = _declared()
    for want in ("fp4mx_quantize", "fp4mx_hadamard_quantize", "fp4mx_gemm", "fp4mx_linear_fwd",
                 "fp4mx_linear_bwd", "fp4nv_quantize46", "fp4nv_gemm", "fp4nv_linear_fwd"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert set(_declared()) == set(binding.EXPORTED)


def test_sign_mask_matches_oracle():
    L = binding.lib()
    for seed in (0, 1, 12345, 2 ** 63 + 7):
        for g in range(3):
            assert L.fp4mx_sign_mask(seed, g) == rng.sign_mask(seed, g)


def test_workspace_sizes():
    L = binding.lib()
    assert L.fp4mx_linear_workspace_bytes(0, 32, 32) == 0
    assert L.fp4mx_linear_workspace_bytes(33, 32, 32) == 0
    m, n, k = 8192, 14336, 4096
    ws = L.fp4mx_linear_workspace_bytes(m, n, k)
    # forward: codes + scales of X and W (4.25 bits/element); backward: dY and dY^T
    assert ws >= max((m * k + n * k) * 17 // 32, 2 * m * n * 17 // 32)
    assert L.fp4mx_ctx_bytes(m, n, k) == (k * m + k * n) * 17 // 32
    assert L.fp4nv_gemm_workspace_bytes(64, 64, 64) >= 2 * 64 * 64 * 33 // 32


def _buf(n=4096):
    b = C.create_string_buffer(n + 64)
    addr = (C.addressof(b) + 63) & ~63
    return b, C.c_void_p(addr)


@pytest.mark.parametrize("case", ["null", "shape", "ld", "align", "round", "axis"])
def test_quantize_validation(case):
    L = binding.lib()
    keep, p = _buf()
    args = dict(x=p, rows=64, cols=64, ld=64, axis=0, rnd=0, codes=p, scales=p)
    want = {"null": -1, "shape": -2, "ld": -3, "align": -3, "round": -4, "axis": -4}[case]
    if case == "null":
        args["x"] = None
    elif case == "shape":
        args["cols"] = 48
    elif case == "ld":
        args["ld"] = 68
    elif case == "align":
        args["codes"] = C.c_void_p(p.value + 4)
    elif case == "round":
        args["rnd"] = 5
    elif case == "axis":
        args["axis"] = 3
    st = L.fp4mx_quantize(args["x"], args["rows"], args["cols"], args["ld"], args["axis"], args["rnd"],
                          0, 0, args["codes"], args["scales"], None)
    assert st == want
    assert L.fp4mx_status_string(st)


def test_maximum_dimension_rejected():
    """Dimensions (and a GEMM's output ldc) above 2^21 are refused before any
    launch: the GEMM's per-tile buffer ranges must stay within 2^31 bytes."""
    L = binding.lib()
    keep, p = _buf()
    f = C.c_void_p(p.value)
    big = (1 << 21) + 32
    assert L.fp4mx_quantize(p, 64, big, big, 0, 0, 0, 0, p, p, None) == -2
    assert L.fp4mx_quantize(p, big, 64, 64, 1, 0, 0, 0, p, p, None) == -2
    assert L.fp4mx_gemm(p, p, p, p, 64, 64, big, 1.0, f, 64, None) == -2
    assert L.fp4mx_gemm(p, p, p, p, big, 64, 64, 1.0, f, 64, None) == -2
    assert L.fp4mx_gemm(p, p, p, p, 64, 64, 64, 1.0, f, big, None) == -2      # ldc above the maximum
    assert L.fp4mx_gemm_bf16(p, p, p, p, 64, 64, 64, 1.0, f, big, None) == -2
    assert L.fp4nv_linear_fwd(p, p, 64, 64, big, f, p, 1 << 20, None) == -2
    assert L.fp4mx_linear_workspace_bytes(64, 64, big) == 0
    assert b"2^21" in L.fp4mx_status_string(-2)


def test_gemm_and_linear_validation():
    L = binding.lib()
    keep, p = _buf()
    f = C.c_void_p(p.value)
    assert L.fp4mx_gemm(p, p, p, p, 64, 64, 0, 1.0, f, 64, None) == -2
    assert L.fp4mx_gemm(p, p, p, p, 64, 64, 64, 1.0, f, 60, None) == -2      # ldc < n
    assert L.fp4mx_gemm(None, p, p, p, 64, 64, 64, 1.0, f, 64, None) == -1
    assert L.fp4mx_gemm_bf16(p, p, p, p, 64, 64, 64, 1.0, f, 68, None) == -3   # ldc not a multiple of 8
    assert L.fp4mx_gemm_bf16(p, p, p, p, 64, 64, 64, 1.0, None, 64, None) == -1
    assert L.fp4mx_gemm_bf16(p, p, p, p, 64, 96, 64, 1.0, f, 64, None) == -2   # ldc < n
    # workspace too small
    ctx = binding.CtxStruct(p.value, p.value, p.value, p.value, 3)
    assert L.fp4mx_linear_fwd(p, p, 64, 64, 64, 3, f, C.byref(ctx), p, 16, None) == -5
    # context seed must match the call's seed
    assert L.fp4mx_linear_fwd(p, p, 64, 64, 64, 4, f, C.byref(ctx), p, 1 << 20, None) == -4
    assert L.fp4mx_linear_bwd(p, None, 64, 64, 64, f, f, p, 1 << 20, None) == -1
    assert L.fp4nv_quantize46(p, 64, 64, 64, 2, p, p, f, p, 256, None) == -4
    assert L.fp4nv_linear_fwd(p, p, 64, 64, 64, f, p, 0, None) == -5


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libfp4mx.so")
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError):
        binding.lib()


def test_quest_validation():
    L = binding.lib()
    keep, p = _buf()
    f = C.c_void_p(p.value)
    m4 = C.c_void_p(p.value + 4)
    assert L.fp4mx_quest_quantize(p, 64, 64, 64, 2.9, 0, p, p, None, None) == -1
    assert L.fp4mx_quest_quantize(p, 64, 64, 64, 2.9, 0, p, p, C.c_void_p(p.value + 2), None) == -3
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert L.fp4mx_quest_quantize(p, 64, 64, 64, bad, 0, p, p, m4, None) == -4
    assert L.fp4mx_quest_quantize(p, 64, 48, 64, 2.9, 0, p, p, m4, None) == -2
    assert L.fp4mx_requantize(p, p, 64, 40, 1, 0, 0, 0, p, p, None) == -2
    assert L.fp4mx_requantize(p, p, 64, 64, 2, 0, 0, 0, p, p, None) == -4
    assert L.fp4mx_requantize(None, p, 64, 64, 1, 0, 0, 0, p, p, None) == -1
    assert L.fp4mx_unmask_inverse_hadamard(f, 64, 64, 62, p, 0, None) == -2
    assert L.fp4mx_unmask_inverse_hadamard(f, 64, 64, 66, p, 0, None) == -3
    ctx = binding.QuestCtxStruct(p.value, p.value, p.value, p.value, p.value, p.value, 3)
    assert L.fp4mx_quest_linear_fwd(p, p, 64, 64, 64, 2.9, 4, f, C.byref(ctx), None) == -4
    assert L.fp4mx_quest_linear_fwd(p, p, 64, 64, 64, 2.9, 3, f, None, None) == -1
    assert L.fp4mx_quest_linear_bwd(p, C.byref(ctx), 64, 64, 64, f, f, p, 16, None) == -5
    bad = binding.QuestCtxStruct(p.value, p.value, p.value, p.value, p.value + 1, p.value, 3)
    assert L.fp4mx_quest_linear_bwd(p, C.byref(bad), 64, 64, 64, f, f, p, 1 << 20, None) == -3
    m, n, k = 8192, 4096, 4096
    assert L.fp4mx_quest_ctx_bytes(m, n, k) == (m * k + n * k) * 17 // 32 + (m * k + n * k) // 8
    assert L.fp4mx_quest_bwd_workspace_bytes(m, n, k) == (2 * m * n + k * n + k * m) * 17 // 32


def test_nv_requant_and_ctx_validation():
    L = binding.lib()
    keep, p = _buf()
    f = C.c_void_p(p.value)
    assert L.fp4nv_msedn_requantize(p, p, f, 96, 64, 6.0, 0, 1, 6, p, p, f, None, p, 1 << 20, None) == -2
    assert L.fp4nv_msedn_requantize(p, p, f, 128, 64, 0.0, 0, 1, 6, p, p, f, None, p, 1 << 20, None) == -4
    assert L.fp4nv_msedn_requantize(p, p, None, 128, 64, 6.0, 0, 1, 6, p, p, f, None, p, 1 << 20, None) == -1
    assert L.fp4nv_msedn_requantize(p, p, f, 128, 64, 6.0, 0, 1, 6, p, p, f, None, p, 16, None) == -5
    ctx = binding.NvCtxStruct(p.value, p.value, p.value, p.value, p.value, p.value, 0)
    assert L.fp4nv_linear_fwd_ctx(p, p, 64, 64, 64, f, C.byref(ctx), p, 16, None) == -5
    assert L.fp4nv_linear_bwd_ctx(p, C.byref(ctx), 128, 96, 64, f, f, p, 1 << 26, None) == -2
    bad = binding.NvCtxStruct(p.value, p.value + 1, p.value, p.value, p.value, p.value, 0)
    assert L.fp4nv_linear_bwd_ctx(p, C.byref(bad), 128, 128, 64, f, f, p, 1 << 26, None) == -3
    assert L.fp4nv_linear_bwd_ctx(p, None, 128, 128, 64, f, f, p, 1 << 26, None) == -1


def test_non_gfx950_device_is_refused():
    """FP4MX_DEVICE_ARCH stands in for the device query: with another
    architecture every compute call returns FP4MX_E_DEVICE after validating
    its arguments and before any HIP call, so this runs without a GPU.  A
    fresh process reads the variable."""
    import subprocess
    import sys
    prog = r'''
import ctypes as C, sys
sys.path.insert(0, %r)
from fp4_microscaled_quantized_amd import binding
L = binding.lib()
b = C.create_string_buffer(1 << 16)
p = C.c_void_p((C.addressof(b) + 255) & ~255)
out = [
    L.fp4mx_quantize(p, 64, 64, 64, 0, 0, 0, 0, p, p, None),
    L.fp4mx_gemm(p, p, p, p, 64, 64, 64, C.c_float(1.0), p, 64, None),
    L.fp4nv_quantize46(p, 64, 64, 64, 1, p, p, p, p, 256, None),
    L.fp4mx_quantize(None, 64, 64, 64, 0, 0, 0, 0, p, p, None),   # validation still first
]
print(" ".join(str(v) for v in out))
''' % ROOT
    env = dict(os.environ, FP4MX_DEVICE_ARCH="gfx942")
    r = subprocess.run([sys.executable, "-c", prog], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["-6", "-6", "-6", "-1"]
    assert binding.lib().fp4mx_status_string(-6) == b"device is not gfx950"


def test_noalloc_rejects_inputs_beyond_its_scratch():
    """fp4nv_msedn_quantize_noalloc checks its static scratch bound on the
    host, after the argument checks and before touching a device."""
    L = binding.lib()
    keep, p = _buf()
    f = lambda r, c, x=p: L.fp4nv_msedn_quantize_noalloc(x, r, c, c, 0, 6.0, 0, 1, 5, p, p, p, None, None)
    assert f(16384, 8192 + 128) == -8          # one 128-chunk per row beyond 2^27 elements
    assert f(32768, 8192) == -8
    assert f(64, 128, None) == -1               # argument checks come first
    assert L.fp4mx_status_string(-8).startswith(b"input needs more scratch")
