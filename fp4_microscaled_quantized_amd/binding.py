"""Thin ctypes binding over libfp4mx.so (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Loading fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4mx.so")

RTN, SR = 0, 1
ROW, COL = 0, 1
# QuEST clip factor: the minimiser over [1, 5] of E[(x - Q_c(clamp(x, -c, c)))^2]
# for x ~ N(0,1), Q_c = E2M1 round-to-nearest on the grid scaled by c/6.
QUEST_CLIP = 2.922475

_lib = None

_P = C.c_void_p
_I64 = C.c_int64
_U32 = C.c_uint32
_U64 = C.c_uint64
_INT = C.c_int
_SZ = C.c_size_t


class CtxStruct(C.Structure):
    _fields_ = [("xt_codes", _P), ("xt_scales", _P), ("wt_codes", _P), ("wt_scales", _P),
                ("seed", _U64)]


class QuestCtxStruct(C.Structure):
    _fields_ = [("xq_codes", _P), ("xq_scales", _P), ("wq_codes", _P), ("wq_scales", _P),
                ("x_mask", _P), ("w_mask", _P), ("seed", _U64)]


class NvCtxStruct(C.Structure):
    _fields_ = [("xq_codes", _P), ("xq_scales", _P), ("xq_tensor_scale", _P), ("wq_codes", _P),
                ("wq_scales", _P), ("wq_tensor_scale", _P), ("seed", _U64)]


_SIGS = {
    "fp4mx_status_string": (C.c_char_p, [_INT]),
    "fp4mx_last_hip_error": (_INT, []),
    "fp4mx_sign_mask": (_U32, [_U64, _U32]),
    "fp4mx_quantize": (_INT, [_P, _I64, _I64, _I64, _INT, _INT, _U64, _U32, _P, _P, _P]),
    "fp4mx_hadamard_quantize": (_INT, [_P, _I64, _I64, _I64, _INT, _INT, _U32, _U64, _U32, _P, _P, _P]),
    "fp4mx_hadamard_quantize_dual": (_INT, [_P, _I64, _I64, _I64, _INT, _U32, _U32, _INT, _U32, _U32,
                                            _U64, _P, _P, _P, _P, _P]),
    "fp4mx_gemm": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, C.c_float, _P, _I64, _P]),
    "fp4mx_gemm_bf16": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, C.c_float, _P, _I64, _P]),
    "fp4mx_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4mx_ctx_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4mx_linear_fwd": (_INT, [_P, _P, _I64, _I64, _I64, _U64, _P, C.POINTER(CtxStruct), _P, _SZ, _P]),
    "fp4mx_linear_bwd": (_INT, [_P, C.POINTER(CtxStruct), _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "fp4mx_linear_fwd_bf16": (_INT, [_P, _P, _I64, _I64, _I64, _U64, _P, C.POINTER(CtxStruct), _P, _SZ,
                                     _P]),
    "fp4mx_linear_bwd_bf16": (_INT, [_P, C.POINTER(CtxStruct), _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "fp4mx_quest_quantize": (_INT, [_P, _I64, _I64, _I64, C.c_float, _U32, _P, _P, _P, _P]),
    "fp4mx_requantize": (_INT, [_P, _P, _I64, _I64, _INT, _U32, _U64, _U32, _P, _P, _P]),
    "fp4mx_unmask_inverse_hadamard": (_INT, [_P, _I64, _I64, _I64, _P, _U32, _P]),
    "fp4mx_gemm_unmask_irht": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, C.c_float, _P, _I64, _P, _U32, _P]),
    "fp4mx_quest_ctx_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4mx_quest_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4mx_quest_linear_fwd": (_INT, [_P, _P, _I64, _I64, _I64, C.c_float, _U64, _P,
                                      C.POINTER(QuestCtxStruct), _P]),
    "fp4mx_quest_linear_bwd": (_INT, [_P, C.POINTER(QuestCtxStruct), _I64, _I64, _I64, _P, _P, _P, _SZ,
                                      _P]),
    "fp4nv_quantize_workspace_bytes": (_SZ, [_I64, _I64]),
    "fp4nv_quantize46": (_INT, [_P, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _SZ, _P]),
    "fp4nv_gemm": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _SZ, _P]),
    "fp4nv_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4nv_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4nv_linear_fwd": (_INT, [_P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "fp4nv_sr_quantize": (_INT, [_P, _I64, _I64, _I64, _U64, _U32, _P, _P, _P, _P, _SZ, _P]),
    "fp4nv_msedn_workspace_bytes": (_SZ, [_I64, _I64]),
    "fp4nv_msedn_quantize": (_INT, [_P, _I64, _I64, _I64, _INT, C.c_float, _U64, _U32, _U32, _P, _P,
                                    _P, _P, _P, _SZ, _P]),
    "fp4nv_msedn_quantize_noalloc": (_INT, [_P, _I64, _I64, _I64, _INT, C.c_float, _U64, _U32, _U32, _P,
                                            _P, _P, _P, _P]),
    "fp4nv_linear_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4nv_linear_bwd": (_INT, [_P, _P, _P, _I64, _I64, _I64, _U64, _P, _P, _P, _SZ, _P]),
    "fp4nv_msedn_requantize": (_INT, [_P, _P, _P, _I64, _I64, C.c_float, _U64, _U32, _U32, _P, _P, _P,
                                      _P, _P, _SZ, _P]),
    "fp4nv_ctx_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4nv_linear_fwd_ctx_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4nv_linear_fwd_ctx": (_INT, [_P, _P, _I64, _I64, _I64, _P, C.POINTER(NvCtxStruct), _P, _SZ, _P]),
    "fp4nv_linear_bwd_ctx": (_INT, [_P, C.POINTER(NvCtxStruct), _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
}

EXPORTED = tuple(_SIGS)


def lib():
    """Load libfp4mx.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4mx.so is not built: run python -m fp4_microscaled_quantized_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class Fp4mxError(RuntimeError):
    pass


def _check(status: int):
    if status != 0:
        L = lib()
        msg = L.fp4mx_status_string(status).decode()
        if status == -7:
            msg += " (hip error %d)" % L.fp4mx_last_hip_error()
        raise Fp4mxError("fp4mx status %d: %s" % (status, msg))


def _ptr(t: torch.Tensor):
    return C.c_void_p(t.data_ptr())


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bf16_2d(x: torch.Tensor):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("expected a 2-D bfloat16 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("innermost dimension must be contiguous")
    return x.shape[0], x.shape[1], x.stride(0)


def sign_mask(seed: int, gemm_id: int) -> int:
    return int(lib().fp4mx_sign_mask(seed, gemm_id))


@dataclass
class MXTensor:
    """An MXFP4 operand: codes [rows, cols/2] uint8, scales [rows, cols/32] uint8."""
    codes: torch.Tensor
    scales: torch.Tensor


def _alloc_mx(rows, cols, device):
    return MXTensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                    torch.empty((rows, cols // 32), dtype=torch.uint8, device=device))


def quantize(x, axis=ROW, rounding=RTN, seed=0, rng_stream=0, hadamard=False, mask=0) -> MXTensor:
    """(RHT +) MXFP4 quantization of a bf16 matrix; COL returns the transposed operand."""
    R, Cc, ld = _bf16_2d(x)
    out = _alloc_mx(R, Cc, x.device) if axis == ROW else _alloc_mx(Cc, R, x.device)
    L = lib()
    if hadamard:
        st = L.fp4mx_hadamard_quantize(_ptr(x), R, Cc, ld, axis, rounding, mask, seed, rng_stream,
                                       _ptr(out.codes), _ptr(out.scales), _stream(x.device))
    else:
        st = L.fp4mx_quantize(_ptr(x), R, Cc, ld, axis, rounding, seed, rng_stream,
                              _ptr(out.codes), _ptr(out.scales), _stream(x.device))
    _check(st)
    return out


def hadamard_quantize(x, axis=ROW, rounding=RTN, mask=0, seed=0, rng_stream=0) -> MXTensor:
    return quantize(x, axis, rounding, seed, rng_stream, hadamard=True, mask=mask)


def hadamard_quantize_dual(x, row_rounding, row_mask, row_stream, col_rounding, col_mask,
                           col_stream, seed=0):
    R, Cc, ld = _bf16_2d(x)
    ro, co = _alloc_mx(R, Cc, x.device), _alloc_mx(Cc, R, x.device)
    _check(lib().fp4mx_hadamard_quantize_dual(
        _ptr(x), R, Cc, ld, row_rounding, row_mask, row_stream, col_rounding, col_mask, col_stream,
        seed, _ptr(ro.codes), _ptr(ro.scales), _ptr(co.codes), _ptr(co.scales), _stream(x.device)))
    return ro, co


def gemm(a: MXTensor, b: MXTensor, alpha: float = 1.0, out: torch.Tensor | None = None):
    """C = alpha * deq(A) deq(B)^T, fp32."""
    m, n, k = a.codes.shape[0], b.codes.shape[0], a.codes.shape[1] * 2
    if b.codes.shape[1] * 2 != k:
        raise ValueError("inner dimensions differ")
    c = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=a.codes.device)
    _check(lib().fp4mx_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), m, n, k,
                            alpha, _ptr(c), c.stride(0), _stream(c.device)))
    return c


def gemm_bf16(a: MXTensor, b: MXTensor, alpha: float = 1.0, out: torch.Tensor | None = None):
    """C = bf16_RNE(alpha * deq(A) deq(B)^T) from the fp32 accumulation."""
    m, n, k = a.codes.shape[0], b.codes.shape[0], a.codes.shape[1] * 2
    if b.codes.shape[1] * 2 != k:
        raise ValueError("inner dimensions differ")
    c = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=a.codes.device)
    if c.dtype != torch.bfloat16:
        raise TypeError("out must be bfloat16")
    _check(lib().fp4mx_gemm_bf16(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), m, n,
                                 k, alpha, _ptr(c), c.stride(0), _stream(c.device)))
    return c


@dataclass
class LinearCtx:
    xt: MXTensor
    wt: MXTensor
    seed: int

    def as_struct(self):
        return CtxStruct(self.xt.codes.data_ptr(), self.xt.scales.data_ptr(),
                         self.wt.codes.data_ptr(), self.wt.scales.data_ptr(), self.seed)


def workspace(m, n, k, device):
    nbytes = lib().fp4mx_linear_workspace_bytes(m, n, k)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _out_entry(dtype, f32_name, bf16_name):
    if dtype == torch.float32:
        return getattr(lib(), f32_name)
    if dtype == torch.bfloat16:
        return getattr(lib(), bf16_name)
    raise ValueError("output dtype must be float32 or bfloat16")


def linear_fwd(x, w, seed=0, want_ctx=True, ws=None, out=None, dtype=torch.float32):
    """Y = X W^T (fp32, or bf16 with dtype=torch.bfloat16) and, when asked,
    the backward context."""
    m, k, _ = _bf16_2d(x)
    n, k2, _ = _bf16_2d(w)
    if k2 != k or not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x [m,k], w [n,k] contiguous")
    fn = _out_entry(dtype, "fp4mx_linear_fwd", "fp4mx_linear_fwd_bf16")
    dev = x.device
    ws = ws if ws is not None else workspace(m, n, k, dev)
    y = out if out is not None else torch.empty((m, n), dtype=dtype, device=dev)
    if y.dtype != dtype or not y.is_contiguous() or tuple(y.shape) != (m, n):
        raise ValueError("out must be a contiguous [m, n] tensor of the output dtype")
    ctx = None
    cs = None
    if want_ctx:
        ctx = LinearCtx(_alloc_mx(k, m, dev), _alloc_mx(k, n, dev), seed)
        cs = C.byref(ctx.as_struct())
    _check(fn(_ptr(x), _ptr(w), m, n, k, seed, _ptr(y), cs, _ptr(ws), ws.numel(), _stream(dev)))
    return y, ctx


def linear_bwd(dy, ctx: LinearCtx, ws=None, dx=None, dw=None, dtype=torch.float32):
    """dX = 16/9 Q(dY) Q(W^T)^T, dW = 16/9 Q(dY^T) Q(X^T)^T (fp32, or bf16
    with dtype=torch.bfloat16)."""
    m, n, _ = _bf16_2d(dy)
    k = ctx.xt.codes.shape[0]
    if not dy.is_contiguous():
        raise ValueError("dy must be contiguous")
    fn = _out_entry(dtype, "fp4mx_linear_bwd", "fp4mx_linear_bwd_bf16")
    dev = dy.device
    ws = ws if ws is not None else workspace(m, n, k, dev)
    dx = dx if dx is not None else torch.empty((m, k), dtype=dtype, device=dev)
    dw = dw if dw is not None else torch.empty((n, k), dtype=dtype, device=dev)
    for t, shp in ((dx, (m, k)), (dw, (n, k))):
        if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError("dx [m, k] and dw [n, k] must be contiguous tensors of the output dtype")
    st = ctx.as_struct()
    _check(fn(_ptr(dy), C.byref(st), m, n, k, _ptr(dx), _ptr(dw), _ptr(ws), ws.numel(), _stream(dev)))
    return dx, dw


# ------------------------------ QuEST --------------------------------------

def quest_quantize(x, clip=QUEST_CLIP, mask=0):
    """QuEST MXFP4 quantization along rows after the RHT: (MXTensor, clip mask [rows, cols/8])."""
    R, Cc, ld = _bf16_2d(x)
    out = _alloc_mx(R, Cc, x.device)
    m = torch.empty((R, Cc // 8), dtype=torch.uint8, device=x.device)
    _check(lib().fp4mx_quest_quantize(_ptr(x), R, Cc, ld, float(clip), mask, _ptr(out.codes),
                                      _ptr(out.scales), _ptr(m), _stream(x.device)))
    return out, m


def requantize(a: MXTensor, rounding=SR, mask=0, seed=0, rng_stream=0) -> MXTensor:
    """Dequantize an MXFP4 operand [rows, cols], transpose, RHT along rows and
    quantize again: the operand [cols, rows]."""
    rows, cols = a.codes.shape[0], a.codes.shape[1] * 2
    out = _alloc_mx(cols, rows, a.codes.device)
    _check(lib().fp4mx_requantize(_ptr(a.codes), _ptr(a.scales), rows, cols, rounding, mask, int(seed),
                                  rng_stream, _ptr(out.codes), _ptr(out.scales),
                                  _stream(a.codes.device)))
    return out


def unmask_inverse_hadamard(c, clip_mask, mask=0):
    """In place: c <- H^-1(c with clipped entries zeroed), per 32-group along rows."""
    if c.dtype != torch.float32 or c.dim() != 2 or c.stride(1) != 1:
        raise ValueError("c must be a row-major fp32 matrix")
    _check(lib().fp4mx_unmask_inverse_hadamard(_ptr(c), c.shape[0], c.shape[1], c.stride(0),
                                               _ptr(clip_mask), mask, _stream(c.device)))
    return c


def gemm_unmask_irht(a: MXTensor, b: MXTensor, clip_mask, alpha: float = 1.0, mask=0, out=None):
    """C = H^-1((alpha deq(A) deq(B)^T) with clipped entries zeroed), fp32, in one kernel."""
    m, n, k = a.codes.shape[0], b.codes.shape[0], a.codes.shape[1] * 2
    if b.codes.shape[1] * 2 != k:
        raise ValueError("inner dimensions differ")
    c = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=a.codes.device)
    _check(lib().fp4mx_gemm_unmask_irht(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), m,
                                        n, k, alpha, _ptr(c), c.stride(0), _ptr(clip_mask), mask,
                                        _stream(c.device)))
    return c


@dataclass
class QuestCtx:
    xq: MXTensor
    wq: MXTensor
    x_mask: torch.Tensor
    w_mask: torch.Tensor
    seed: int

    def as_struct(self):
        return QuestCtxStruct(self.xq.codes.data_ptr(), self.xq.scales.data_ptr(),
                              self.wq.codes.data_ptr(), self.wq.scales.data_ptr(),
                              self.x_mask.data_ptr(), self.w_mask.data_ptr(), self.seed)


def quest_linear_fwd(x, w, seed=0, clip=QUEST_CLIP, ctx=None, out=None):
    """Y = X_q W_q^T with QuEST operands; returns (Y fp32, QuestCtx)."""
    m, k, _ = _bf16_2d(x)
    n, k2, _ = _bf16_2d(w)
    if k2 != k or not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x [m,k], w [n,k] contiguous")
    dev = x.device
    if ctx is None:
        ctx = QuestCtx(_alloc_mx(m, k, dev), _alloc_mx(n, k, dev),
                       torch.empty((m, k // 8), dtype=torch.uint8, device=dev),
                       torch.empty((n, k // 8), dtype=torch.uint8, device=dev), seed)
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    st = ctx.as_struct()
    _check(lib().fp4mx_quest_linear_fwd(_ptr(x), _ptr(w), m, n, k, float(clip), seed, _ptr(y),
                                        C.byref(st), _stream(dev)))
    return y, ctx


def quest_linear_bwd(dy, ctx: QuestCtx, ws=None, dx=None, dw=None):
    """dX, dW in the forward-rotated basis with mask correction and inverse RHT (fp32)."""
    m, n, _ = _bf16_2d(dy)
    k = ctx.xq.codes.shape[1] * 2
    if not dy.is_contiguous():
        raise ValueError("dy must be contiguous")
    dev = dy.device
    if ws is None:
        ws = torch.empty(lib().fp4mx_quest_bwd_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    dx = dx if dx is not None else torch.empty((m, k), dtype=torch.float32, device=dev)
    dw = dw if dw is not None else torch.empty((n, k), dtype=torch.float32, device=dev)
    st = ctx.as_struct()
    _check(lib().fp4mx_quest_linear_bwd(_ptr(dy), C.byref(st), m, n, k, _ptr(dx), _ptr(dw), _ptr(ws),
                                        ws.numel(), _stream(dev)))
    return dx, dw


# ------------------------------ NVFP4 --------------------------------------

@dataclass
class NVTensor:
    """NVFP4 operand: codes [rows, cols/2], E4M3 scales [rows, cols/16], fp32 tensor scale [1]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor


def nv_quantize46(x, use_46=True) -> NVTensor:
    R, Cc, ld = _bf16_2d(x)
    dev = x.device
    out = NVTensor(torch.empty((R, Cc // 2), dtype=torch.uint8, device=dev),
                   torch.empty((R, Cc // 16), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev))
    ws = torch.empty(lib().fp4nv_quantize_workspace_bytes(R, Cc), dtype=torch.uint8, device=dev)
    _check(lib().fp4nv_quantize46(_ptr(x), R, Cc, ld, int(use_46), _ptr(out.codes), _ptr(out.scales),
                                  _ptr(out.tensor_scale), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def nv_gemm(a: NVTensor, b: NVTensor, ws=None):
    m, n, k = a.codes.shape[0], b.codes.shape[0], a.codes.shape[1] * 2
    dev = a.codes.device
    if ws is None:
        ws = torch.empty(lib().fp4nv_gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    _check(lib().fp4nv_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale), _ptr(b.codes),
                            _ptr(b.scales), _ptr(b.tensor_scale), m, n, k, _ptr(c), n, _ptr(ws),
                            ws.numel(), _stream(dev)))
    return c


def nv_linear_fwd(x, w, ws=None, out=None):
    m, k, _ = _bf16_2d(x)
    n, _, _ = _bf16_2d(w)
    dev = x.device
    if ws is None:
        ws = torch.empty(lib().fp4nv_linear_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    _check(lib().fp4nv_linear_fwd(_ptr(x), _ptr(w), m, n, k, _ptr(y), _ptr(ws), ws.numel(),
                                  _stream(dev)))
    return y


def nv_sr_quantize(x, seed=0, stream=1) -> NVTensor:
    """Standard NVFP4 stochastic rounding (16/17 guard) of x along rows."""
    R, Cc, ld = _bf16_2d(x)
    dev = x.device
    out = NVTensor(torch.empty((R, Cc // 2), dtype=torch.uint8, device=dev),
                   torch.empty((R, Cc // 16), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev))
    ws = torch.empty(lib().fp4nv_quantize_workspace_bytes(R, Cc), dtype=torch.uint8, device=dev)
    _check(lib().fp4nv_sr_quantize(_ptr(x), R, Cc, ld, int(seed), stream, _ptr(out.codes),
                                   _ptr(out.scales), _ptr(out.tensor_scale), _ptr(ws), ws.numel(),
                                   _stream(dev)))
    return out


def nv_msedn_quantize(x, axis=ROW, seed=0, gemm_id=1, stream=5, clip=6.0, want_s=False):
    """MS-EDEN of x (bf16 2-D): NVTensor of the output operand ([rows, cols]
    for ROW, [cols, rows] for COL), plus S per 128-chunk when want_s."""
    R, Cc, ld = _bf16_2d(x)
    dev = x.device
    orow, ocol = (R, Cc) if axis == ROW else (Cc, R)
    out = NVTensor(torch.empty((orow, ocol // 2), dtype=torch.uint8, device=dev),
                   torch.empty((orow, ocol // 16), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev))
    s_out = torch.empty((orow, ocol // 128), dtype=torch.float32, device=dev) if want_s else None
    ws = torch.empty(lib().fp4nv_msedn_workspace_bytes(R, Cc), dtype=torch.uint8, device=dev)
    _check(lib().fp4nv_msedn_quantize(_ptr(x), R, Cc, ld, axis, float(clip), int(seed), gemm_id, stream,
                                      _ptr(out.codes), _ptr(out.scales), _ptr(out.tensor_scale),
                                      _ptr(s_out) if want_s else None, _ptr(ws), ws.numel(), _stream(dev)))
    return (out, s_out) if want_s else out


def nv_linear_bwd(dy, x, w, seed=0, ws=None, dx=None, dw=None):
    """NVFP4 backward with MS-EDEN operands: (dX [m,k], dW [n,k]) fp32."""
    m, n, _ = _bf16_2d(dy)
    _, k, _ = _bf16_2d(x)
    dev = dy.device
    if ws is None:
        ws = torch.empty(lib().fp4nv_linear_bwd_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    dx = dx if dx is not None else torch.empty((m, k), dtype=torch.float32, device=dev)
    dw = dw if dw is not None else torch.empty((n, k), dtype=torch.float32, device=dev)
    _check(lib().fp4nv_linear_bwd(_ptr(dy), _ptr(x), _ptr(w), m, n, k, int(seed), _ptr(dx), _ptr(dw),
                                  _ptr(ws), ws.numel(), _stream(dev)))
    return dx, dw


def nv_msedn_requantize(a: "NVTensor", seed=0, gemm_id=1, stream=6, clip=6.0, want_s=False):
    """MS-EDEN of the transpose of a saved NVFP4 operand [rows, cols] -> [cols, rows]."""
    rows, cols = a.codes.shape[0], a.codes.shape[1] * 2
    dev = a.codes.device
    out = NVTensor(torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev),
                   torch.empty((cols, rows // 16), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev))
    s_out = torch.empty((cols, rows // 128), dtype=torch.float32, device=dev) if want_s else None
    ws = torch.empty(lib().fp4nv_msedn_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    _check(lib().fp4nv_msedn_requantize(_ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale), rows, cols,
                                        float(clip), int(seed), gemm_id, stream, _ptr(out.codes),
                                        _ptr(out.scales), _ptr(out.tensor_scale),
                                        _ptr(s_out) if want_s else None, _ptr(ws), ws.numel(), _stream(dev)))
    return (out, s_out) if want_s else out


@dataclass
class NvCtx:
    """Saved forward operands of the NVFP4 layer and the backward seed."""
    xq: "NVTensor"
    wq: "NVTensor"
    seed: int

    def as_struct(self):
        return NvCtxStruct(self.xq.codes.data_ptr(), self.xq.scales.data_ptr(),
                           self.xq.tensor_scale.data_ptr(), self.wq.codes.data_ptr(),
                           self.wq.scales.data_ptr(), self.wq.tensor_scale.data_ptr(), self.seed)


def _alloc_nv(rows, cols, dev):
    return NVTensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                    torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
                    torch.empty(1, dtype=torch.float32, device=dev))


def nv_linear_fwd_ctx(x, w, seed=0, ws=None, out=None):
    """NVFP4 forward (RTN + 4/6) keeping Q(X), Q(W): (Y fp32, NvCtx)."""
    m, k, _ = _bf16_2d(x)
    n, _, _ = _bf16_2d(w)
    dev = x.device
    ctx = NvCtx(_alloc_nv(m, k, dev), _alloc_nv(n, k, dev), seed)
    if ws is None:
        ws = torch.empty(lib().fp4nv_linear_fwd_ctx_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    st = ctx.as_struct()
    _check(lib().fp4nv_linear_fwd_ctx(_ptr(x), _ptr(w), m, n, k, _ptr(y), C.byref(st), _ptr(ws), ws.numel(),
                                      _stream(dev)))
    return y, ctx


def nv_linear_bwd_ctx(dy, ctx: NvCtx, ws=None, dx=None, dw=None):
    """NVFP4 backward re-quantizing the saved Q(X), Q(W) with MS-EDEN: (dX, dW) fp32."""
    m, n, _ = _bf16_2d(dy)
    k = ctx.xq.codes.shape[1] * 2
    dev = dy.device
    if ws is None:
        ws = torch.empty(lib().fp4nv_linear_bwd_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    dx = dx if dx is not None else torch.empty((m, k), dtype=torch.float32, device=dev)
    dw = dw if dw is not None else torch.empty((n, k), dtype=torch.float32, device=dev)
    st = ctx.as_struct()
    _check(lib().fp4nv_linear_bwd_ctx(_ptr(dy), C.byref(st), m, n, k, _ptr(dx), _ptr(dw), _ptr(ws),
                                      ws.numel(), _stream(dev)))
    return dx, dw


# --------------------------- autograd wrapper --------------------------------

class FP4LinearFunction(torch.autograd.Function):
    """Y = X W^T with all three GEMMs in MXFP4, for bf16 X and W.

    Y, dX and dW come out of the library as bf16 (the GEMMs' bf16 epilogue:
    round to nearest even of the fp32 result), so no cast runs outside it."""

    @staticmethod
    def forward(ctx, x, w, seed):
        if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
            raise TypeError("FP4LinearFunction takes bf16 x and w")
        y, c = linear_fwd(x.contiguous(), w.contiguous(), seed=int(seed), want_ctx=True,
                          dtype=torch.bfloat16)
        ctx.fp4 = c
        return y

    @staticmethod
    def backward(ctx, gy):
        if gy.dtype != torch.bfloat16:
            raise TypeError("FP4LinearFunction expects a bf16 output gradient")
        dx, dw = linear_bwd(gy.contiguous(), ctx.fp4, dtype=torch.bfloat16)
        return dx, dw, None
