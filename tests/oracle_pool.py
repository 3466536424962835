"""Full-size oracle evaluation for the parity tests, split over worker processes.

The oracle's quantizers treat output rows independently: an MXFP4 row (or a
column of the input, for the column axis) depends only on its own 32-groups,
and the SR draws are indexed by the row's global index, which ``row_ids``
passes in.  The NVFP4 quantizer needs the tensor's global scale, computed once
here and passed to every chunk.  Splitting the output rows across processes
therefore computes exactly what one call over the whole tensor computes; it
only lets the full-size checks finish in seconds.

Workers are spawned (fresh interpreters that import numpy and the oracle only;
they never touch the GPU).  This module imports no torch.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os

import numpy as np

from oracle import mx, nvfp4

WORKERS = max(1, min(12, os.cpu_count() or 1))
_pool = None


def pool():
    global _pool
    if _pool is None:
        _pool = mp.get_context("spawn").Pool(WORKERS)
        atexit.register(_shutdown)
    return _pool


def _shutdown():
    global _pool
    if _pool is not None:
        _pool.terminate()
        _pool.join()
        _pool = None


def _split(n: int, parts: int):
    b = np.linspace(0, n, parts + 1).astype(np.int64)
    return [(int(b[i]), int(b[i + 1])) for i in range(parts) if b[i + 1] > b[i]]


def _mx_chunk(args):
    x, kw, row_ids = args
    return mx.quantize(x, row_ids=row_ids, **kw)


def mx_quantize(x: np.ndarray, *, rounding, axis=mx.ROW, hadamard=True, sign_mask=0, seed=0,
                stream=0, rows=None):
    """``mx.quantize`` over the whole operand (or only output rows ``rows``, a
    sorted index array), evaluated in row chunks."""
    x = np.asarray(x, dtype=np.float32)
    n_out = x.shape[0] if axis == mx.ROW else x.shape[1]
    ids = np.arange(n_out) if rows is None else np.asarray(rows, dtype=np.int64)
    kw = dict(rounding=rounding, axis=axis, hadamard=hadamard, sign_mask=sign_mask, seed=seed,
              stream=stream)
    tasks = []
    for a, b in _split(ids.size, 4 * WORKERS):
        sel = ids[a:b]
        part = x[sel] if axis == mx.ROW else np.ascontiguousarray(x[:, sel])
        tasks.append((part, kw, sel))
    parts = pool().map(_mx_chunk, tasks)
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def _nv_chunk(args):
    x, use46, g = args
    c, s, _ = nvfp4.quantize46(x, use46, g=g)
    return c, s


def nv_quantize46(x: np.ndarray, use46: bool = True, rows=None):
    """``nvfp4.quantize46`` of the whole tensor (its global scale from all of
    x), evaluated in row chunks; ``rows`` restricts the output rows."""
    x = np.asarray(x, dtype=np.float32)
    g = nvfp4.tensor_scale(x)
    ids = np.arange(x.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    tasks = [(x[ids[a:b]], use46, g) for a, b in _split(ids.size, 4 * WORKERS)]
    parts = pool().map(_nv_chunk, tasks)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), g


def _stage_chunk(args):
    codes, scales = args
    return nvfp4.fp8_stage_bytes(codes, scales)


def nv_fp8_stage(codes: np.ndarray, scales: np.ndarray):
    """``nvfp4.fp8_stage_bytes`` (row-independent) evaluated in row chunks."""
    tasks = [(codes[a:b], scales[a:b]) for a, b in _split(codes.shape[0], 4 * WORKERS)]
    parts = pool().map(_stage_chunk, tasks)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
