#!/usr/bin/env python3
"""Benchmark of the fully-FP4 (MXFP4) linear layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
forward (RHT + RTN quantization of X and W fused with the SR context, FP4
GEMM Y = X W^T) and backward (RHT + SR quantization of dY and dY^T, FP4 GEMMs
dX and dW): fp4mx_linear_fwd + fp4mx_linear_bwd through the C ABI.  The timed
steps run back to back with HIP events at step boundaries only (value,
ms_per_step).  The same kernels are then launched one by one through the
single-operation entry points with an event after every launch, which gives
each kernel's in-step duration (breakdown_ms), and the three GEMMs back to
back give the GEMM roofline.

Headline workload: Quartet-style layer, 8192 tokens, d_in = d_out = 4096.
value = 6*M*N*K flop / step time (TFLOP/s).  Printed as one JSON line.

Extra fields (same line): the Llama-3-8B FFN-up layer (8192 x 4096 -> 14336),
the stand-alone quantizer on the 8192 x 4096 workload (GB/s, HBM roofline,
rotating input buffers so the 256 MB Infinity Cache cannot hold them), the
NVFP4 forward variant (16384 x 8192 -> 8192), and the CPU oracle timed on a
bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 linear fwd+bwd TFLOPS (% FP4 MFMA peak); quantizer GB/s (% HBM)"
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# vector ALU issue: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz, one 64-lane wave
# instruction per SIMD every 4 cycles (a transcendental takes 12 more)
PEAK_VALU_TLANE = 256 * 4 * 16 * 2.4e9 / 1e12
MX_BYTES_PER_ELEM = 2 + 0.5 + 1 / 32   # bf16 in, 4-bit code + 1/32 scale byte out
ROTATE_BYTES = 1 << 30                  # linear-layer inputs in rotation: at least 1 GiB
DIST_STEPS = 200                        # steps timed one by one for the median


_T0 = time.time()


def progress(msg):
    """One progress line on stderr (stdout carries only the JSON result)."""
    print("[bench %6.1f s] %s" % (time.time() - _T0, msg), file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["quartet", "llama"], default="quartet")
    p.add_argument("--no-extra", action="store_true", help="only the headline workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--dist-steps", type=int, default=DIST_STEPS,
                   help="steps timed one by one for the step-time distribution (0: none)")
    p.add_argument("--vendor", action="store_true",
                   help="also time hipBLASLt's MXFP4 GEMM beside the kernel (its set-up takes minutes)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one 512 MiB device copy (traffic counter calibration)")
    return p.parse_args()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class _Step:
    """A sequence of C-ABI launches on one stream, timed per step and per launch."""

    def _step_calls(self):
        """Launch lists, one per input set (step i uses set i % nsets)."""
        return [self._calls(i) for i in range(getattr(self, "nsets", 1))]

    def _part_calls(self):
        """The step's kernels launched one by one, as `names` lists them (for
        the per-launch breakdown and the GEMM pass); by default the step's
        own launches."""
        return self._step_calls()

    def run(self, steps, timed):
        """`steps` passes of the launches, back to back; when timed, one event
        before the first and one after the last launch (nothing is inserted
        between steps or kernels)."""
        import torch
        sc = self._step_calls()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if timed else None
        if timed:
            evs[0].record()
        for i in range(steps):
            for c in sc[i % len(sc)]:
                c()
        if timed:
            evs[1].record()
        return evs

    def step_times(self, steps):
        """Duration of each of `steps` back-to-back steps: one event at every
        step boundary (ms per step, a list)."""
        import torch
        sc = self._step_calls()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            for c in sc[i % len(sc)]:
                c()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]

    def group_time(self, idx, steps, warmup):
        """Mean time of one pass over the launches idx of `_part_calls` (the
        step's kernels and buffers), `steps` passes back to back between one
        event pair after `warmup` untimed passes: ms per pass."""
        import torch
        sc = self._part_calls()
        for i in range(warmup):
            for j in idx:
                sc[i % len(sc)][j]()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for i in range(steps):
            for j in idx:
                sc[i % len(sc)][j]()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    def kernel_times(self, steps):
        """In-step duration of each launch: the step's kernels one by one
        (`_part_calls`), `steps` passes with an event after every launch, all
        on the stream the kernels run on (an event record adds a few
        microseconds to the launch it follows)."""
        import torch
        sc = self._part_calls()
        evs = []
        for s_ in range(steps):
            calls = sc[s_ % len(sc)]
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
            ev[0].record()
            for i, c in enumerate(calls):
                c()
                ev[i + 1].record()
            evs.append(ev)
        torch.cuda.synchronize()
        for ev in evs:
            for i, nm in enumerate(self.names):
                self.times[nm].append(ev[i].elapsed_time(ev[i + 1]))

    def flops(self):
        return 6.0 * self.m * self.n * self.k


class LinearStep(_Step):
    """The MXFP4 linear fwd+bwd hot path: a step is fp4mx_linear_fwd (with the
    backward context) + fp4mx_linear_bwd on one stream.  The same kernels
    launched one by one through the single-operation entry points (six
    launches: X and W quantized separately, where fp4mx_linear_fwd quantizes
    both in one launch) give the per-launch breakdown and the GEMM pass."""

    def __init__(self, d, seed=0, rotate_bytes=ROTATE_BYTES):
        import torch
        import fp4_microscaled_quantized_amd as fq
        self.fq = fq
        x, w, dy = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
        # input sets in rotation: step i reads set i % nsets, and the sets
        # together exceed the 256 MB Infinity Cache several times over, so a
        # step's inputs come from HBM (copies hold the same values)
        per_set = (x.numel() + w.numel() + dy.numel()) * 2
        self.nsets = max(1, -(-rotate_bytes // per_set))
        self.sets = [(x, w, dy)] + [(x.clone(), w.clone(), dy.clone()) for _ in range(self.nsets - 1)]
        self.x, self.w, self.dy = x, w, dy
        self.rotating_MB = round(self.nsets * per_set / 1e6, 1)
        self.m, self.k = self.x.shape
        self.n = self.w.shape[0]
        self.seed = seed
        m, n, k = self.m, self.n, self.k
        dev = self.x.device
        e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
        self.xq, self.xs, self.xtq, self.xts = e(m, k // 2), e(m, k // 32), e(k, m // 2), e(k, m // 32)
        self.wq, self.wsc, self.wtq, self.wts = e(n, k // 2), e(n, k // 32), e(k, n // 2), e(k, n // 32)
        self.dq, self.ds, self.dtq, self.dts = e(m, n // 2), e(m, n // 32), e(n, m // 2), e(n, m // 32)
        f = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        self.y, self.dx, self.dw = f(m, n), f(m, k), f(n, k)
        # the layer entry points' own outputs, context and workspace
        self.ly, self.ldx, self.ldw = f(m, n), f(m, k), f(n, k)
        self.lctx = fq.LinearCtx(fq.binding._alloc_mx(k, m, dev), fq.binding._alloc_mx(k, n, dev), seed)
        self.lctx_struct = self.lctx.as_struct()
        self.ws = fq.binding.workspace(m, n, k, dev)
        self.g = [fq.sign_mask(seed, i) for i in range(3)]
        self.names = ["quant_x", "quant_w", "gemm_y", "quant_dy", "gemm_dx", "gemm_dw"]
        self.times = {nm: [] for nm in self.names}

    def _calls(self, i=0):
        """One step: fp4mx_linear_fwd with the context, then fp4mx_linear_bwd."""
        import ctypes
        L = self.fq.lib()
        from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
        s = _stream()
        m, n, k, seed = self.m, self.n, self.k, self.seed
        x, w, dy = self.sets[i % self.nsets]
        cs = ctypes.byref(self.lctx_struct)
        return [
            lambda: _check(L.fp4mx_linear_fwd(_ptr(x), _ptr(w), m, n, k, seed, _ptr(self.ly), cs,
                                              _ptr(self.ws), self.ws.numel(), s)),
            lambda: _check(L.fp4mx_linear_bwd(_ptr(dy), cs, m, n, k, _ptr(self.ldx), _ptr(self.ldw),
                                              _ptr(self.ws), self.ws.numel(), s)),
        ]

    def _part_calls(self):
        return [self._parts(i) for i in range(self.nsets)]

    def _parts(self, i=0):
        """The step's kernels launched one by one, in `names` order."""
        fq, L = self.fq, self.fq.lib()
        from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
        s = _stream()
        m, n, k, seed = self.m, self.n, self.k, self.seed
        g0, g1, g2 = self.g
        RTN, SR = fq.RTN, fq.SR
        x, w, dy = self.sets[i % self.nsets]
        return [
            lambda: _check(L.fp4mx_hadamard_quantize_dual(_ptr(x), m, k, k, RTN, g0, 0, SR, g2, 4, seed,
                                                          _ptr(self.xq), _ptr(self.xs), _ptr(self.xtq),
                                                          _ptr(self.xts), s)),
            lambda: _check(L.fp4mx_hadamard_quantize_dual(_ptr(w), n, k, k, RTN, g0, 0, SR, g1, 2, seed,
                                                          _ptr(self.wq), _ptr(self.wsc), _ptr(self.wtq),
                                                          _ptr(self.wts), s)),
            lambda: _check(L.fp4mx_gemm(_ptr(self.xq), _ptr(self.xs), _ptr(self.wq), _ptr(self.wsc), m, n, k,
                                        1.0, _ptr(self.y), n, s)),
            lambda: _check(L.fp4mx_hadamard_quantize_dual(_ptr(dy), m, n, n, SR, g1, 1, SR, g2, 3, seed,
                                                          _ptr(self.dq), _ptr(self.ds), _ptr(self.dtq),
                                                          _ptr(self.dts), s)),
            lambda: _check(L.fp4mx_gemm(_ptr(self.dq), _ptr(self.ds), _ptr(self.wtq), _ptr(self.wts), m, k, n,
                                        16.0 / 9.0, _ptr(self.dx), k, s)),
            lambda: _check(L.fp4mx_gemm(_ptr(self.dtq), _ptr(self.dts), _ptr(self.xtq), _ptr(self.xts), n, k, m,
                                        16.0 / 9.0, _ptr(self.dw), k, s)),
        ]

    def check_against_composite(self):
        """The launches one by one must reproduce the layer entry points' step
        bit for bit (outputs and context)."""
        import torch
        for c in self._parts(0) + self._calls(0):
            c()
        torch.cuda.synchronize()
        lc = self.lctx
        ok = (torch.equal(self.ly, self.y) and torch.equal(self.ldx, self.dx) and torch.equal(self.ldw, self.dw)
              and torch.equal(lc.xt.codes, self.xtq) and torch.equal(lc.xt.scales, self.xts)
              and torch.equal(lc.wt.codes, self.wtq) and torch.equal(lc.wt.scales, self.wts))
        if not ok:
            raise SystemExit("the launches one by one differ from fp4mx_linear_fwd/bwd")



class QuestStep(_Step):
    """QuEST forward + the Quartet backward in the forward-rotated basis as eight
    C-ABI launches: QuEST X, QuEST W, GEMM Y, dual SR quant dY, re-quantize
    W_q and X_q, GEMM dX and GEMM dW with the mask + inverse-RHT epilogue."""

    def __init__(self, d, seed=0):
        import torch
        import fp4_microscaled_quantized_amd as fq
        self.fq = fq
        self.x, self.w, self.dy = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
        self.m, self.k = self.x.shape
        self.n = self.w.shape[0]
        self.seed = seed
        m, n, k = self.m, self.n, self.k
        dev = self.x.device
        e = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
        self.xq, self.xs, self.xm = e(m, k // 2), e(m, k // 32), e(m, k // 8)
        self.wq, self.wsc, self.wm = e(n, k // 2), e(n, k // 32), e(n, k // 8)
        self.xtq, self.xts, self.wtq, self.wts = e(k, m // 2), e(k, m // 32), e(k, n // 2), e(k, n // 32)
        self.dq, self.ds, self.dtq, self.dts = e(m, n // 2), e(m, n // 32), e(n, m // 2), e(n, m // 32)
        f = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        self.y, self.dx, self.dw = f(m, n), f(m, k), f(n, k)
        self.g = [fq.sign_mask(seed, i) for i in range(3)]
        self.names = ["quest_x", "quest_w", "gemm_y", "quant_dy", "requant_w", "requant_x",
                      "gemm_dx_irht", "gemm_dw_irht"]
        self.times = {nm: [] for nm in self.names}

    def _calls(self, i=0):
        fq, L = self.fq, self.fq.lib()
        from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
        s = _stream()
        m, n, k, seed = self.m, self.n, self.k, self.seed
        g0, g1, g2 = self.g
        c = float(fq.QUEST_CLIP)
        SR = fq.SR
        a = 16.0 / 9.0
        return [
            lambda: _check(L.fp4mx_quest_quantize(_ptr(self.x), m, k, k, c, g0, _ptr(self.xq), _ptr(self.xs),
                                                  _ptr(self.xm), s)),
            lambda: _check(L.fp4mx_quest_quantize(_ptr(self.w), n, k, k, c, g0, _ptr(self.wq), _ptr(self.wsc),
                                                  _ptr(self.wm), s)),
            lambda: _check(L.fp4mx_gemm(_ptr(self.xq), _ptr(self.xs), _ptr(self.wq), _ptr(self.wsc), m, n, k,
                                        1.0, _ptr(self.y), n, s)),
            lambda: _check(L.fp4mx_hadamard_quantize_dual(_ptr(self.dy), m, n, n, SR, g1, 1, SR, g2, 3, seed,
                                                          _ptr(self.dq), _ptr(self.ds), _ptr(self.dtq),
                                                          _ptr(self.dts), s)),
            lambda: _check(L.fp4mx_requantize(_ptr(self.wq), _ptr(self.wsc), n, k, SR, g1, seed, 2,
                                              _ptr(self.wtq), _ptr(self.wts), s)),
            lambda: _check(L.fp4mx_requantize(_ptr(self.xq), _ptr(self.xs), m, k, SR, g2, seed, 4,
                                              _ptr(self.xtq), _ptr(self.xts), s)),
            lambda: _check(L.fp4mx_gemm_unmask_irht(_ptr(self.dq), _ptr(self.ds), _ptr(self.wtq), _ptr(self.wts),
                                                    m, k, n, a, _ptr(self.dx), k, _ptr(self.xm), g0, s)),
            lambda: _check(L.fp4mx_gemm_unmask_irht(_ptr(self.dtq), _ptr(self.dts), _ptr(self.xtq),
                                                    _ptr(self.xts), n, k, m, a, _ptr(self.dw), k, _ptr(self.wm),
                                                    g0, s)),
        ]

    def check_against_composite(self):
        """The decomposed calls must reproduce fp4mx_quest_linear_fwd / _bwd bit for bit."""
        import torch
        fq = self.fq
        self.run(1, False)
        y, ctx = fq.quest_linear_fwd(self.x, self.w, seed=self.seed)
        dx, dw = fq.quest_linear_bwd(self.dy, ctx)
        torch.cuda.synchronize()
        ok = (torch.equal(y, self.y) and torch.equal(dx, self.dx) and torch.equal(dw, self.dw)
              and torch.equal(ctx.x_mask, self.xm) and torch.equal(ctx.wq.scales, self.wsc))
        if not ok:
            raise SystemExit("decomposed QuEST step differs from fp4mx_quest_linear_fwd/bwd")


def time_step(st, steps, warmup, dist_steps=0):
    """Optionally `dist_steps` steps with an event at every step boundary (the
    distribution; they also bring the clocks to their steady state), then
    the warm-up, then `steps` timed steps (wall clock and one event pair),
    then the per-kernel pass."""
    import torch
    st.check_against_composite()
    dist = st.step_times(dist_steps) if dist_steps else None
    st.run(warmup, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = st.run(steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [evs[0].elapsed_time(evs[1]) / steps]
    st.kernel_times(steps)
    avg = {nm: float(np.mean(v)) for nm, v in st.times.items()}
    return wall, avg, step_ms, dist


def time_quest(steps, warmup):
    """The QuEST layer on the Quartet workload: step rate and each quantizer
    against its roofline (algorithmic bytes: QuEST 2 + 0.5 + 1/32 + 1/8 B per
    element, re-quantizer 2 x 0.53125)."""
    from fp4_microscaled_quantized_amd import synth
    st = QuestStep(synth.quartet_linear(0))
    wall, avg, _, _ = time_step(st, steps, warmup)
    ms = wall * 1e3 / steps
    m, n, k = st.m, st.n, st.k
    by = {"quest_x": m * k * (2 + 0.5 + 1 / 32 + 1 / 8), "quest_w": n * k * (2 + 0.5 + 1 / 32 + 1 / 8),
          "requant_w": n * k * 2 * (0.5 + 1 / 32), "requant_x": m * k * 2 * (0.5 + 1 / 32)}
    kr = {nm: {"GB/s": round(b / (avg[nm] * 1e-3) / 1e9, 1),
               "frac_hbm": round(b / (avg[nm] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)} for nm, b in by.items()}
    gemm_ms = avg["gemm_y"] + avg["gemm_dx_irht"] + avg["gemm_dw_irht"]
    return {"workload": "QuEST fwd + Quartet bwd (rotated basis; masks and inverse RHT in the GEMM epilogue) "
                        "M=8192 N=K=4096",
            "ms_per_step": round(ms, 4), "TFLOP/s": round(st.flops() / (ms * 1e-3) / 1e12, 1),
            "gemm_TFLOP/s": round(6.0 * m * n * k / (gemm_ms * 1e-3) / 1e12, 1),
            "breakdown_ms": {nm: round(v, 4) for nm, v in avg.items()}, "kernel_hbm": kr}


def time_linear(d, steps, warmup, seed=0, dist_steps=0):
    st = LinearStep(d, seed)
    wall, avg, step_ms, dist = time_step(st, steps, warmup, dist_steps)
    # the three GEMMs of the step back to back (no event between launches)
    st.gemm_pass_ms = st.group_time([2, 4, 5], steps, warmup)
    return st, wall, avg, step_ms, dist


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "mx_gemm_kernel_quartet_8192x4096x4096_traffic.json")


def gemm_traffic(st):
    """Mean HBM bytes per GEMM launch from the committed FETCH_SIZE / WRITE_SIZE
    record (copy-calibrated), if it was taken on this exact kernel source and
    workload; None otherwise."""
    import hashlib
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    if sha != rec["source_sha256"] or "%dx%dx%d" % (st.m, st.n, st.k) != rec["workload"]:
        return None
    b = rec["bytes_per_launch"]
    return int(round(np.mean([b["gemm_y"], b["gemm_dx"], b["gemm_dw"]])))


def gemm_roofline(st, avg):
    """FP4 MFMA roofline of the GEMM kernel: 2MNK flop per launch / mean launch
    time, the time from the step's three GEMMs run back to back between one
    event pair (an event after every launch, as in `avg`, adds a few
    microseconds to each)."""
    m, n, k = st.m, st.n, st.k
    fl = {"gemm_y": 2.0 * m * n * k, "gemm_dx": 2.0 * m * k * n, "gemm_dw": 2.0 * n * k * m}
    tot_fl = sum(fl.values())
    tot_ms = st.gemm_pass_ms
    achieved = tot_fl / (tot_ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": "mx_gemm_kernel (FP4 32x32x64 scaled MFMA)",
            "achieved": round(achieved, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP4_TFLOPS, 4), "traffic": gemm_traffic(st),
            "traffic_unit": "bytes per launch (HBM/fabric, FETCH_SIZE + WRITE_SIZE)",
            "algorithmic_bytes_per_launch": int(round(np.mean(
                [(m + n) * k * 17 // 32 + 4 * m * n, (m + k) * n * 17 // 32 + 4 * m * k,
                 (n + k) * m * 17 // 32 + 4 * n * k]))),
            "mean_launch_ms": round(tot_ms / 3, 4),
            "mean_launch_timing": "the three GEMMs of the step, K passes back to back, one event pair",
            "per_launch_ms": {x: round(avg[x], 4) for x in fl},
            "per_launch_timing": "in the step, an event after every launch"}


def mfma_sustained(fmt=4, iters=20000, reps=3):
    """Sustained rate of the GEMMs' scaled MFMA (fmt 4: FP4 x FP4, 0: FP8 E4M3
    x FP8) on this GPU, measured with libfp4mx_probe.so (16 independent MFMAs
    per iteration per wave, one workgroup of 4 waves per CU, no memory traffic
    in the loop), with random operand bits and with all-zero operands, and the
    shader clock of the run (shader-clock counter over the 100-MHz reference
    counter)."""
    import ctypes
    import torch
    from fp4_microscaled_quantized_amd import build as fbuild
    lib = ctypes.CDLL(fbuild.PROBE_LIB)
    lib.fp4mx_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    blocks = 256
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda").manual_seed(7)
    rnd = torch.randint(-2 ** 31, 2 ** 31 - 1, (4096,), dtype=torch.int32, device="cuda", generator=g)
    if fmt == 0:
        # E4M3 bytes with the NaN encodings (0x7f, 0xff) replaced by the largest finite value
        b = rnd.view(torch.uint8).clone()
        b[(b & 0x7f) == 0x7f] -= 1
        rnd = b.view(torch.int32)
    words = {"random_operands": rnd, "zero_operands": torch.zeros(4096, dtype=torch.int32, device="cuda")}
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    flops = blocks * 4.0 * iters * 16 * 2 * 32 * 32 * 64
    out = {"probe": "v_mfma_scale_f32_32x32x64_f8f6f4, %s, %d workgroups x 4 waves x %d x 16 MFMAs"
                    % ("FP4 x FP4" if fmt == 4 else "FP8 E4M3 x E4M3", blocks, iters)}
    for kind, w in words.items():
        def call(i):
            st_ = lib.fp4mx_probe_mfma(fmt, w.data_ptr(), iters, blocks, sink.data_ptr(), clk.data_ptr(), stream)
            if st_ != 0:
                raise RuntimeError("MFMA probe launch failed: %d" % st_)
        ms = _time_calls(call, reps, 1)
        c = clk.cpu().numpy().astype(np.uint64)
        ghz = float(c[1] - c[0]) / (float(c[3] - c[2]) / 100e6) / 1e9
        out[kind] = {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "clock_GHz": round(ghz, 3)}
    return out


def quant_roofline(st, avg):
    m, n, k = st.m, st.n, st.k
    # dual quantizer: 2 B read + two outputs of 0.5 + 1/32 B per element
    by = {"quant_x": m * k * (2 + 2 * (0.5 + 1 / 32)), "quant_w": n * k * (2 + 2 * (0.5 + 1 / 32)),
          "quant_dy": m * n * (2 + 2 * (0.5 + 1 / 32))}
    gbs = sum(by.values()) / (sum(avg[x] for x in by) * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


QUANT_VALU_RECORD = os.path.join(ROOT, "profiles", "quantizer_in_step_valu_record.json")


def quant_alu_roofline(st, avg):
    """ALU roofline of the step's three quantizer launches: the VALU
    instructions each issues (committed SQ_INSTS_VALU / SQ_INSTS_VALU_TRANS_F32
    record, taken on this exact quantizer source and workload) against the
    chip's vector issue rate; None when the record does not match."""
    import hashlib
    try:
        with open(QUANT_VALU_RECORD) as f:
            rec = json.load(f)
        for src, sha in rec["source_sha256"].items():
            with open(os.path.join(ROOT, src), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != sha:
                    return None
    except (OSError, ValueError, KeyError):
        return None
    if "%dx%dx%d" % (st.m, st.n, st.k) != rec["workload"]:
        return None
    keys = ("quant_x", "quant_w", "quant_dy")
    lane_instr = sum(64.0 * (rec["valu_per_launch"][x] + 3.0 * rec["trans_per_launch"][x]) for x in keys)
    t = sum(avg[x] for x in keys) * 1e-3
    ach = lane_instr / t / 1e12
    return {"bound": "alu", "achieved": round(ach, 2), "peak": round(PEAK_VALU_TLANE, 2),
            "unit": "T VALU lane-instructions/s (a transcendental counts 4)",
            "frac": round(ach / PEAK_VALU_TLANE, 4),
            "valu_per_launch": {x: rec["valu_per_launch"][x] for x in keys},
            "record": os.path.relpath(QUANT_VALU_RECORD, ROOT)}


def time_quantizer(steps, warmup, nbuf=6):
    """fp4mx_hadamard_quantize (row axis) on the 8192 x 4096 workload, RTN and SR."""
    import torch
    import fp4_microscaled_quantized_amd as fq
    from fp4_microscaled_quantized_amd import synth
    from fp4_microscaled_quantized_amd.binding import _check, _ptr, _stream
    x0 = dev_bf16(synth.quantizer_tensor()["x"])
    R, Cc = x0.shape
    xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
    outs = [(torch.empty((R, Cc // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((R, Cc // 32), dtype=torch.uint8, device="cuda")) for _ in range(nbuf)]
    L = fq.lib()
    mask = fq.sign_mask(0, 0)
    res = {}
    outs_t = [(torch.empty((Cc, R // 2), dtype=torch.uint8, device="cuda"),
               torch.empty((Cc, R // 32), dtype=torch.uint8, device="cuda")) for _ in range(nbuf)]
    for name, rnd, axis in (("rtn", fq.RTN, fq.ROW), ("sr", fq.SR, fq.ROW),
                            ("rtn_col", fq.RTN, fq.COL), ("sr_col", fq.SR, fq.COL)):
        o = outs if axis == fq.ROW else outs_t

        def call(i, rnd=rnd, axis=axis, o=o):
            _check(L.fp4mx_hadamard_quantize(_ptr(xs[i % nbuf]), R, Cc, Cc, axis, rnd, mask, 0, 1,
                                             _ptr(o[i % nbuf][0]), _ptr(o[i % nbuf][1]), _stream()))
        # back-to-back launches, events only around the whole run
        ms = _time_calls(call, steps, warmup)
        byt = R * Cc * MX_BYTES_PER_ELEM
        gbs = byt / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": int(byt)}
    # context: a plain device copy of the same bf16 tensor (read + write 2 B per
    # element) over the same rotating buffers, i.e. what streaming reaches at this size
    ys = [torch.empty_like(x0) for _ in range(nbuf)]
    cms = _time_calls(lambda i: ys[i % nbuf].copy_(xs[i % nbuf]), steps, warmup)
    res["copy_bf16_GB/s"] = round(R * Cc * 4 / (cms * 1e-3) / 1e9, 1)
    return {"workload": "quantizer 8192x4096 bf16, half N(0,1) half Student-t(3), RHT-32; row axis "
                        "(rtn, sr) and column axis, i.e. the transposed operand (rtn_col, sr_col)",
            "rotating_buffers_MB": round(nbuf * (R * Cc * 2 + R * Cc * 17 // 32) / 1e6, 1), **res}


def time_nvfp4(steps, warmup):
    import torch
    import fp4_microscaled_quantized_amd as fq
    from fp4_microscaled_quantized_amd import synth
    d = synth.nvfp4_linear(0)
    x, w = dev_bf16(d["x"]), dev_bf16(d["w"])
    m, k = x.shape
    n = w.shape[0]
    ws = torch.empty(fq.lib().fp4nv_linear_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        fq.nv_linear_fwd(x, w, ws=ws, out=y)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        fq.nv_linear_fwd(x, w, ws=ws, out=y)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    # the quantizer (tensor amax pass + RTN/4-over-6 pass) on X alone
    from fp4_microscaled_quantized_amd.binding import _ptr, _stream
    L = fq.lib()
    qc = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((m, k // 16), dtype=torch.uint8, device="cuda")
    qg = torch.empty(1, dtype=torch.float32, device="cuda")
    qws = torch.empty(L.fp4nv_quantize_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    qcall = lambda i: L.fp4nv_quantize46(_ptr(x), m, k, k, 1, _ptr(qc), _ptr(qs), _ptr(qg), _ptr(qws),
                                         qws.numel(), _stream())
    assert qcall(0) == 0
    qms = _time_calls(qcall, max(steps, 10), 2)
    two = m * k * (2 + 2 + 0.5 + 1 / 16)
    one = m * k * (2 + 0.5 + 1 / 16)
    return {"workload": "NVFP4 RTN+4/6 linear fwd 16384x8192->8192", "ms": round(ms, 4),
            "TFLOP/s": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "quantizer_x_16384x8192": {"us": round(qms * 1e3, 1),
                                       "GB/s_two_pass_bytes": round(two / (qms * 1e-3) / 1e9, 1),
                                       "frac_hbm_two_pass": round(two / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                       "GB/s_one_read_bytes": round(one / (qms * 1e-3) / 1e9, 1)}}


def _time_calls(call, steps, warmup):
    import torch
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(steps):
        call(i)
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def time_gemm_outputs(steps, warmup, rounds=3):
    """The MXFP4 GEMM with fp32 output against the bf16-output variant
    (fp4mx_gemm_bf16), per launch, on the Quartet and Llama FFN-up shapes.
    The two are timed alternately, `rounds` times each; medians reported."""
    import torch
    import fp4_microscaled_quantized_amd as fq
    res = {"workload": "MXFP4 GEMM per launch, fp32 vs bf16 output (random codes, E8M0 scales 2^-9..2^2)"}
    for (m, n, k) in [(8192, 4096, 4096), (8192, 14336, 4096)]:
        g = torch.Generator(device="cuda").manual_seed(5)

        def op(r):
            return fq.MXTensor(torch.randint(0, 256, (r, k // 2), dtype=torch.uint8, device="cuda", generator=g),
                               torch.randint(118, 130, (r, k // 32), dtype=torch.uint8, device="cuda", generator=g))
        A, B = op(m), op(n)
        c32 = torch.empty((m, n), dtype=torch.float32, device="cuda")
        c16 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        t32, t16 = [], []
        for _ in range(rounds):
            t32.append(_time_calls(lambda i: fq.gemm(A, B, out=c32), steps, warmup))
            t16.append(_time_calls(lambda i: fq.gemm_bf16(A, B, out=c16), steps, warmup))
        t32, t16 = float(np.median(t32)), float(np.median(t16))
        fl = 2.0 * m * n * k
        res["%dx%dx%d" % (m, n, k)] = {"fp32_out_us": round(t32 * 1e3, 1), "bf16_out_us": round(t16 * 1e3, 1),
                                        "fp32_out_TFLOP/s": round(fl / (t32 * 1e-3) / 1e12, 1),
                                        "bf16_out_TFLOP/s": round(fl / (t16 * 1e-3) / 1e12, 1)}
        del A, B, c32, c16
        torch.cuda.empty_cache()
    return res


def _vendor_lib():
    import ctypes as C
    from fp4_microscaled_quantized_amd import binding
    L = C.CDLL(os.path.join(os.path.dirname(binding.LIB_PATH), "libfp4mx_vendor.so"))
    L.fp4mx_vendor_plan_create.restype = C.c_int
    L.fp4mx_vendor_plan_create.argtypes = [C.c_int64] * 3 + [C.POINTER(C.c_void_p), C.POINTER(C.c_int)]
    L.fp4mx_vendor_gemm.restype = C.c_int
    L.fp4mx_vendor_gemm.argtypes = [C.c_void_p, C.c_int] + [C.c_void_p] * 4 + [C.c_float, C.c_void_p, C.c_void_p]
    L.fp4mx_vendor_plan_destroy.restype = None
    L.fp4mx_vendor_plan_destroy.argtypes = [C.c_void_p]
    return L


def time_vendor_gemm(steps, warmup, rounds=3):
    """hipBLASLt's MXFP4 GEMM (libfp4mx_vendor.so) beside fp4mx_gemm on the
    same random operands and the same stream: the fastest of the heuristic
    algorithms hipBLASLt offers (each timed over `steps` calls), then the two
    timed alternately `rounds` times; medians.  The outputs' relative
    Frobenius difference is reported as a sanity check."""
    import ctypes as C
    import torch
    import fp4_microscaled_quantized_amd as fq
    from fp4_microscaled_quantized_amd.binding import _stream
    try:
        V = _vendor_lib()
    except OSError as e:
        return {"unavailable": str(e)}
    res = {"workload": "MXFP4 GEMM per launch, fp32 output, random codes and E8M0 scales 2^-9..2^3; "
                       "hipBLASLt: VEC32_UE8M0 block scales, fastest of its heuristic algorithms"}
    for (m, n, k) in [(8192, 4096, 4096), (8192, 14336, 4096)]:
        key = "%dx%dx%d" % (m, n, k)
        plan, nalg = C.c_void_p(), C.c_int()
        st = V.fp4mx_vendor_plan_create(m, n, k, C.byref(plan), C.byref(nalg))
        progress("  hipBLASLt plan %s: status %d, %d algorithms" % (key, st, nalg.value))
        if st != 0:
            res[key] = {"unavailable": "no hipBLASLt MXFP4 algorithm (status %d)" % st}
            continue
        try:
            g = torch.Generator(device="cuda").manual_seed(11)

            def padded(rows, cols, lo, hi):
                t = torch.randint(lo, hi, (rows * cols + (1 << 20),), dtype=torch.uint8, device="cuda", generator=g)
                return t[:rows * cols].view(rows, cols)
            a, as_ = padded(m, k // 2, 0, 256), padded(m, k // 32, 118, 131)
            b, bs = padded(n, k // 2, 0, 256), padded(n, k // 32, 118, 131)
            A, B = fq.MXTensor(a, as_), fq.MXTensor(b, bs)
            c0 = torch.empty((m, n), dtype=torch.float32, device="cuda")
            c1 = torch.empty((m, n), dtype=torch.float32, device="cuda")
            s = _stream(c1.device)

            def vend(al):
                return lambda i: V.fp4mx_vendor_gemm(plan, al, a.data_ptr(), as_.data_ptr(), b.data_ptr(),
                                                     bs.data_ptr(), 1.0, c1.data_ptr(), s)
            per_algo = []
            for al in range(nalg.value):
                if vend(al)(0) != 0:
                    per_algo.append(float("inf"))
                    continue
                per_algo.append(_time_calls(vend(al), steps, warmup))
                progress("  hipBLASLt algorithm %d: %.1f us" % (al, per_algo[-1] * 1e3))
            best = int(np.argmin(per_algo))
            tv, to = [], []
            for _ in range(rounds):
                to.append(_time_calls(lambda i: fq.gemm(A, B, out=c0), steps, warmup))
                tv.append(_time_calls(vend(best), steps, warmup))
            to, tv = float(np.median(to)), float(np.median(tv))
            torch.cuda.synchronize()
            diff = float(torch.linalg.vector_norm(c1 - c0) / torch.linalg.vector_norm(c0))
            fl = 2.0 * m * n * k
            res[key] = {"fp4mx_us": round(to * 1e3, 1), "hipblaslt_us": round(tv * 1e3, 1),
                        "fp4mx_TFLOP/s": round(fl / (to * 1e-3) / 1e12, 1),
                        "hipblaslt_TFLOP/s": round(fl / (tv * 1e-3) / 1e12, 1),
                        "speedup": round(tv / to, 3), "hipblaslt_algorithms": nalg.value,
                        "hipblaslt_per_algorithm_us": [round(x * 1e3, 1) for x in per_algo],
                        "rel_fro_difference": diff}
            del a, as_, b, bs, A, B, c0, c1
        finally:
            V.fp4mx_vendor_plan_destroy(plan)
        torch.cuda.empty_cache()
    return res


def time_nvfp4_bwd(steps, warmup):
    """NVFP4 backward with MS-EDEN operands on the Quartet layer (dX and dW,
    4 MS-EDEN quantizations + 2 FP8-staged GEMMs), and the unbiased quantizers
    alone on dY (8192 x 4096) against their algorithmic bytes."""
    import torch
    import fp4_microscaled_quantized_amd as fq
    from fp4_microscaled_quantized_amd import synth
    from fp4_microscaled_quantized_amd.binding import _ptr, _stream
    d = synth.quartet_linear(0)
    x, w, dy = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
    m, k = x.shape
    n = w.shape[0]
    L = fq.lib()
    ws = torch.empty(L.fp4nv_linear_bwd_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    dx = torch.empty((m, k), dtype=torch.float32, device="cuda")
    dw = torch.empty((n, k), dtype=torch.float32, device="cuda")
    ms = _time_calls(lambda i: fq.nv_linear_bwd(dy, x, w, seed=i, ws=ws, dx=dx, dw=dw), steps, warmup)
    res = {"workload": "NVFP4 MS-EDEN linear bwd dX,dW M=8192 N=K=4096", "ms": round(ms, 4),
           "TFLOP/s": round(4.0 * m * n * k / (ms * 1e-3) / 1e12, 1)}
    del ws
    R, C = dy.shape
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, C // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    qws = torch.empty(max(L.fp4nv_msedn_workspace_bytes(R, C), L.fp4nv_quantize_workspace_bytes(R, C)),
                      dtype=torch.uint8, device="cuda")
    st = _stream(dy.device)
    alg = R * C * (2 + 0.5 + 1 / 16)  # bf16 in, E2M1 codes + E4M3 scales out
    qs = {}
    for name, call in (
        ("ms_eden_row", lambda i: L.fp4nv_msedn_quantize(_ptr(dy), R, C, C, fq.ROW, 6.0, i, 1, 5, _ptr(codes),
                                                         _ptr(scales), _ptr(g), None, _ptr(qws),
                                                         qws.numel(), st)),
        ("sr_baseline_row", lambda i: L.fp4nv_sr_quantize(_ptr(dy), R, C, C, i, 5, _ptr(codes), _ptr(scales),
                                                          _ptr(g), _ptr(qws), qws.numel(), st))):
        assert call(0) == 0
        qms = _time_calls(call, max(steps, 20), warmup)
        qs[name] = {"us": round(qms * 1e3, 2), "GB/s": round(alg / (qms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(alg / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    res["quantizers_8192x4096"] = qs
    res["quantizer_algorithmic_bytes"] = int(alg)
    return res


def time_quartet2(steps, warmup):
    """The Quartet II graph on the Quartet layer: NVFP4 forward keeping Q(X),
    Q(W) and the backward re-quantizing them with MS-EDEN (6MNK flop per
    step), plus the re-quantizer alone on the saved Q(X) (8192 x 4096) against
    its algorithmic bytes (0.5 + 1/16 B read, 0.5 + 1/16 B written per element)."""
    import torch
    import fp4_microscaled_quantized_amd as fq
    from fp4_microscaled_quantized_amd import synth
    from fp4_microscaled_quantized_amd.binding import _ptr, _stream
    d = synth.quartet_linear(0)
    x, w, dy = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
    m, k = x.shape
    n = w.shape[0]
    L = fq.lib()
    wsf = torch.empty(L.fp4nv_linear_fwd_ctx_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(L.fp4nv_linear_bwd_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.float32, device="cuda")
    dw = torch.empty((n, k), dtype=torch.float32, device="cuda")
    _, ctx = fq.nv_linear_fwd_ctx(x, w, seed=0, ws=wsf, out=y)

    def step(i):
        fq.nv_linear_fwd_ctx(x, w, seed=i, ws=wsf, out=y)
        ctx.seed = i
        fq.nv_linear_bwd_ctx(dy, ctx, ws=wsb, dx=dx, dw=dw)
    ms = _time_calls(step, steps, warmup)
    fwd_ms = _time_calls(lambda i: fq.nv_linear_fwd_ctx(x, w, seed=i, ws=wsf, out=y), steps, warmup)
    res = {"workload": "Quartet II graph: NVFP4 RTN+4/6 fwd (saved Q(X), Q(W)) + MS-EDEN bwd "
                       "re-quantizing them, M=8192 N=K=4096",
           "ms_per_step": round(ms, 4), "TFLOP/s": round(6.0 * m * n * k / (ms * 1e-3) / 1e12, 1),
           "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(ms - fwd_ms, 4)}
    del wsb
    out_c = torch.empty((k, m // 2), dtype=torch.uint8, device="cuda")
    out_s = torch.empty((k, m // 16), dtype=torch.uint8, device="cuda")
    out_g = torch.empty(1, dtype=torch.float32, device="cuda")
    qws = torch.empty(L.fp4nv_msedn_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    st = _stream(x.device)
    xq = ctx.xq
    call = lambda i: L.fp4nv_msedn_requantize(_ptr(xq.codes), _ptr(xq.scales), _ptr(xq.tensor_scale), m, k,
                                              6.0, i, 2, 8, _ptr(out_c), _ptr(out_s), _ptr(out_g), None,
                                              _ptr(qws), qws.numel(), st)
    assert call(0) == 0
    qms = _time_calls(call, max(steps, 20), warmup)
    alg = m * k * 2 * (0.5 + 1 / 16)
    res["requant_q_x"] = {"us": round(qms * 1e3, 2), "GB/s": round(alg / (qms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(alg / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes": int(alg)}
    return res


def _oracle_quant_rows(args):
    """Worker: the oracle's MXFP4 quantizer on a chunk of rows (spawned process)."""
    from oracle import mx
    x, kw, row_ids = args
    return mx.quantize(x, row_ids=row_ids, **kw)


def _cpu_model():
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(rows=1024, target_s=15.0):
    """The oracle on the host's cores.

    value: the oracle's linear fwd+bwd on the first `rows` tokens of the
    headline workload (TFLOP/s).  The time is a fixed part (the weight's
    quantizations) plus a part per row; a 32-row run and a `rows`-row run fit
    the two, and the sample is then sized, in whole 32-row blocks, so that the
    timed run takes about target_s.  NumPy's elementwise work runs on one
    thread, its fp64 matmuls on all BLAS threads.

    full_size: the 8192 x 4096 quantizer (RHT + RTN, 84.9 MB of algorithmic
    traffic) and the 8192 x 4096 x 4096 GEMM (on operands quantized
    beforehand), each at full size, on 1 thread and on all cores (row chunks
    over worker processes for the quantizer, BLAS threads for the GEMM)."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_info, threadpool_limits
    from fp4_microscaled_quantized_amd import synth
    from oracle import mx, rng
    d = synth.quartet_linear(0)
    f = synth.bf16_bits_to_f32
    w = f(d["w"])
    n, k = w.shape
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    workers = max(1, min(16, os.cpu_count() or 1))

    def run(r):
        x, dy = f(d["x"][:r]), f(d["dy"][:r])
        t0 = time.perf_counter()
        y, ctx = mx.linear_fwd(x, w, seed=0)
        mx.linear_bwd(dy, ctx)
        return time.perf_counter() - t0

    t_fix = run(32)
    progress("  oracle 32 rows: %.1f s" % t_fix)
    dt = run(rows)
    progress("  oracle %d rows: %.1f s" % (rows, dt))
    per_row = max(dt - t_fix, 1e-3) / (rows - 32)
    grown = int((target_s - t_fix) / per_row) // 32 * 32
    if grown > rows:
        rows = min(8192, grown)
        dt = run(rows)
        progress("  oracle %d rows: %.1f s" % (rows, dt))
    flop = 6.0 * rows * n * k
    res = {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
           "sample": "linear fwd+bwd on the first %d of 8192 token rows of the 8192x4096x4096 workload "
                     "(6*%d*4096*4096 flop) in %.1f s; numpy elementwise on 1 thread, fp64 matmul on %d "
                     "BLAS threads" % (rows, rows, dt, blas),
           "cpu_model": _cpu_model(), "host_cpus_visible": os.cpu_count()}

    progress("  oracle full-size quantizer and GEMM")
    # full-size quantizer: 8192 x 4096, RHT + RTN (GEMM-0 mask)
    xq = f(synth.quantizer_tensor()["x"])
    R, Cq = xq.shape
    kw = dict(rounding=mx.RTN, sign_mask=rng.sign_mask(0, 0))
    qbytes = R * Cq * (2 + 0.5 + 1 / 32)
    t0 = time.perf_counter()
    mx.quantize(xq, **kw)
    q1 = time.perf_counter() - t0
    bounds = np.linspace(0, R, 4 * workers + 1).astype(int)
    tasks = [(xq[a:b], kw, np.arange(a, b)) for a, b in zip(bounds[:-1], bounds[1:])]
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(_oracle_quant_rows, tasks[:workers])           # start the workers
        t0 = time.perf_counter()
        pool.map(_oracle_quant_rows, tasks)
        qn = time.perf_counter() - t0
        # GEMM operands for the full-size GEMM, quantized in the same pool (untimed)
        x, g0 = f(d["x"]), rng.sign_mask(0, 0)
        gkw = dict(rounding=mx.RTN, sign_mask=g0)
        parts = []
        for src in (x, w):
            b2 = np.linspace(0, src.shape[0], 4 * workers + 1).astype(int)
            ps = pool.map(_oracle_quant_rows, [(src[a:b], gkw, np.arange(a, b)) for a, b in zip(b2[:-1], b2[1:])])
            parts.append((np.concatenate([p[0] for p in ps]), np.concatenate([p[1] for p in ps])))
    gflop = 2.0 * x.shape[0] * n * k
    with threadpool_limits(1):
        t0 = time.perf_counter()
        mx.gemm(*parts[0], *parts[1])
        g1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    mx.gemm(*parts[0], *parts[1])
    gn = time.perf_counter() - t0
    res["full_size"] = {
        "quantizer_8192x4096_rht_rtn": {
            "1_thread": {"s": round(q1, 2), "GB/s": round(qbytes / q1 / 1e9, 4)},
            "all_cores": {"s": round(qn, 2), "GB/s": round(qbytes / qn / 1e9, 4), "processes": workers}},
        "gemm_8192x4096x4096": {
            "1_thread": {"s": round(g1, 2), "TFLOP/s": round(gflop / g1 / 1e12, 5)},
            "all_cores": {"s": round(gn, 2), "TFLOP/s": round(gflop / gn / 1e12, 5), "blas_threads": int(blas)},
            "note": "dequantize to fp64 and one fp64 matmul (the oracle's GEMM)"}}
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from fp4_microscaled_quantized_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if a.calib_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    if a.workload == "quartet":
        d = synth.quartet_linear(0)
        wl = {"workload": "quartet_linear fwd+bwd M=8192 N=4096 K=4096", "m": 8192, "n": 4096, "k": 4096}
    else:
        d = synth.llama_ffn_up(0)
        wl = {"workload": "llama3_8b_ffn_up fwd+bwd M=8192 K=4096 N=14336", "m": 8192, "n": 14336, "k": 4096}
    progress("linear step %s" % wl["workload"])
    st, wall, avg, step_ms, dist = time_linear(d, a.steps, a.warmup,
                                              dist_steps=max(a.steps, a.dist_steps) if a.dist_steps else 0)
    progress("linear step timed: %.4f ms" % (wall * 1e3 / a.steps))
    ev_ms = sum(avg.values())
    ms_step = wall * 1e3 / a.steps
    value = st.flops() / (ms_step * 1e-3) / 1e12
    dist = dist if dist else step_ms
    med = float(np.median(dist))
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic", "config": {**wl, "seed": 0, "parallelism": "none (1 GPU)",
                                        "rotating_input_sets": st.nsets, "rotating_inputs_MB": st.rotating_MB},
        "frac_fp4_peak": round(value / PEAK_FP4_TFLOPS, 4),
        "roofline": gemm_roofline(st, avg),
        "mfma_fp4_sustained": mfma_sustained(4),
        "breakdown_ms": {k2: round(v, 4) for k2, v in avg.items()},
        "breakdown_timing": "the step's kernels launched one by one (X and W quantized in two launches, "
                            "which fp4mx_linear_fwd fuses into one), an event after every launch",
        "kernel_sum_ms_per_step": round(ev_ms, 4),
        "event_ms_per_step": round(float(np.mean(step_ms)), 4),
        "step_distribution": {"steps": len(dist), "median_ms": round(med, 4),
                              "mean_ms": round(float(np.mean(dist)), 4),
                              "p10_ms": round(float(np.percentile(dist, 10)), 4),
                              "p90_ms": round(float(np.percentile(dist, 90)), 4),
                              "median_TFLOP/s": round(st.flops() / (med * 1e-3) / 1e12, 1),
                              "note": "one event at every step boundary, inputs rotating over the sets above"},
        "quantizer_roofline_in_step": quant_roofline(st, avg),
        "quantizer_alu_roofline_in_step": quant_alu_roofline(st, avg),
    }
    sus = out["mfma_fp4_sustained"]["random_operands"]["TFLOP/s"]
    out["roofline"]["sustained_peak_random_operands"] = sus
    out["roofline"]["frac_of_sustained"] = round(out["roofline"]["achieved"] / sus, 4)
    del st
    torch.cuda.empty_cache()
    if not a.no_extra:
        if a.workload == "quartet":
            progress("llama ffn-up step")
            st2, wall2, avg2, _, _ = time_linear(synth.llama_ffn_up(0), a.steps, a.warmup)
            ms2 = wall2 * 1e3 / a.steps
            out["llama_ffn_up"] = {"workload": "8192 x 4096 -> 14336 fwd+bwd", "ms_per_step": round(ms2, 4),
                                   "TFLOP/s": round(st2.flops() / (ms2 * 1e-3) / 1e12, 1),
                                   "gemm_roofline": gemm_roofline(st2, avg2),
                                   "breakdown_ms": {k2: round(v, 4) for k2, v in avg2.items()}}
            del st2
            torch.cuda.empty_cache()
        progress("gemm output dtypes")
        out["gemm_output_dtype"] = time_gemm_outputs(max(a.steps // 2, 20), 10)
        torch.cuda.empty_cache()
        progress("quantizers")
        out["quantizer"] = time_quantizer(max(a.steps, 20), a.warmup)
        torch.cuda.empty_cache()
        progress("nvfp4 forward")
        out["nvfp4"] = time_nvfp4(max(a.steps // 2, 5), 2)
        out["nvfp4"]["mfma_fp8_sustained"] = mfma_sustained(0)
        sus8 = out["nvfp4"]["mfma_fp8_sustained"]["random_operands"]["TFLOP/s"]
        out["nvfp4"]["frac_fp8_sustained"] = round(out["nvfp4"]["TFLOP/s"] / sus8, 4)
        torch.cuda.empty_cache()
        progress("nvfp4 ms-eden backward")
        out["nvfp4_bwd_ms_eden"] = time_nvfp4_bwd(max(a.steps // 2, 5), 2)
        torch.cuda.empty_cache()
        progress("quest layer")
        out["quest_linear"] = time_quest(a.steps, a.warmup)
        torch.cuda.empty_cache()
        progress("quartet ii graph")
        out["nvfp4_quartet2"] = time_quartet2(max(a.steps // 2, 5), 2)
    if a.vendor:
        progress("hipBLASLt MXFP4 gemm")
        out["vendor_gemm"] = time_vendor_gemm(20, 5)
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        progress("cpu baseline (oracle)")
        cb = cpu_baseline()
        # GPU over oracle, the same work on each side (context only)
        sp = {"linear_fwd_bwd_8192x4096x4096": round(value / cb["value"], 1)}
        fs = cb["full_size"]
        if "quantizer" in out:
            q_s = out["quantizer"]["rtn"]["ms"] * 1e-3
            sp["quantizer_8192x4096_rht_rtn"] = {
                "vs_1_thread": round(fs["quantizer_8192x4096_rht_rtn"]["1_thread"]["s"] / q_s, 1),
                "vs_all_cores": round(fs["quantizer_8192x4096_rht_rtn"]["all_cores"]["s"] / q_s, 1)}
        g_s = out["roofline"]["mean_launch_ms"] * 1e-3
        sp["gemm_8192x4096x4096"] = {"vs_1_thread": round(fs["gemm_8192x4096x4096"]["1_thread"]["s"] / g_s, 1),
                                     "vs_all_cores": round(fs["gemm_8192x4096x4096"]["all_cores"]["s"] / g_s, 1)}
        cb["gpu_speedup"] = sp
        out["cpu_baseline"] = cb
    progress("done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
