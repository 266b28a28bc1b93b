#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 hot path on one MI355X.

A step is one pass of a workload's whole path over one batch of seeded
synthetic input already resident in HBM. The headline step (the default) is
the random-Hadamard activation workload, the largest configuration:
NVFP4 four-over-six quantization with the 16-point random Hadamard
transform of the activations X [16384, 4096] and of the weight W [4096,
12288] (quantized transposed), each with its tensor-amax pre-pass, then the
NVFP4 GEMM 16384 x 12288 x 4096 to bf16. The same JSON line carries, under
"workloads", the mixture-of-experts MXFP4 step (32 experts: W^T and X
quantize, grouped GEMM 32 x 512 x 5760 x 2880), the training quantize step
(8192^2 weight with 16 x 16 scales as-is and transposed, gradient with
stochastic rounding) and the W4A4 linear step (2048 x 4096 x 4096), and under
"worked_example" the codes, scales and MAE of the 4096-value example in the
whole-tensor, MXFP4, NVFP4 and four-over-six modes.

Timing: W untimed warm-up steps, then K steps between two device
synchronisations, with HIP events (torch.cuda.Event on the stream the kernels
run on) around every op; the step time is the average over replays of HIP
graphs of the step. Inputs rotate over enough copies (>= 600 MB) that the
256 MB Infinity Cache cannot serve them from one step to the next. Every
NVFP4 quantize is also timed on its own with the tensor amax supplied
(kernel-only), beside its end-to-end time with the pre-pass.

Output: one JSON line. `value` is the step's roofline time (sum over its ops
of algorithmic bytes / 8 TB/s for codec scans, flops / dense matrix peak for
the GEMM) as a percentage of the measured step time. `roofline` describes the
op that takes most of the step; `kernels` lists every op. `cpu_baseline`
times the CPU oracle, as it stands, on a bounded sample of the same workload,
on one core and on all host cores (rows split over processes), scaled to the
full step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import tempfile
import time
from dataclasses import dataclass, field
from pathlib import Path

import numpy as np
import torch

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "FP4 quantize GB/s + W4A4 GEMM TFLOPS, each as % of MI355X roofline"
PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp4": 10100.0}  # dense matrix-core peaks
ROTATE_BYTES = 600 << 20


class Op:
    """One library call in the step: `launch(i)` enqueues it for input set i.
    lane 0: on the step's stream, after every op before it; lane k > 0: on
    side stream k, after the last lane-0 op before it (independent of the
    other lanes' ops since then)."""

    def __init__(self, name, kernel, bound, work, peak, launch, unit, lane=0):
        self.name, self.kernel, self.bound, self.work, self.peak = name, kernel, bound, work, peak
        self.launch, self.unit, self.lane = launch, unit, lane
        self.durations = []

    def roofline_seconds(self):
        return self.work / (self.peak * 1e9 if self.unit == "GB/s" else self.peak * 1e12)


def quant_bytes(elems_in, in_bytes, blk, nv, batch=1):
    return elems_in * in_bytes + elems_in // 2 + elems_in // blk + (4 * batch if nv else 0)


class QuantCall:
    """Preallocated fp4_quantize call over `sets` input copies."""

    def __init__(self, F, xs, fmt, flags=0, signs=0, seed=0, offset=0, amax=None):
        self.F, self.xs = F, xs
        self.amax = amax  # device float[batch] or None (kept alive here)
        x = xs[0]
        x3 = x if x.dim() == 3 else x.unsqueeze(0)
        self.batch, self.rows, self.cols = x3.shape
        tr = bool(flags & F.FP4_TRANSPOSE)
        R, C = (self.cols, self.rows) if tr else (self.rows, self.cols)
        self.R, self.C = R, C
        self.blk = 16 if fmt == F.FP4_NVFP4 else 32
        dev = x.device
        self.opts = F.make_opts(fmt, flags, signs, seed, offset, amax.data_ptr() if amax is not None else 0)
        self.ldc = F.code_pitch(C // 2)  # code rows on whole 128-byte lines
        self.codes = torch.empty((self.batch, R, self.ldc), dtype=torch.uint8, device=dev)[:, :, : C // 2]
        self.lds = F.scale_pitch(C // self.blk)  # scale rows padded to 16 bytes, as the GEMM reads them
        self.scales_buf = torch.empty((self.batch, R, self.lds), dtype=torch.uint8, device=dev)
        self.scales = self.scales_buf[:, :, : C // self.blk]
        self.ts = torch.empty((self.batch,), dtype=torch.float32, device=dev)
        self.ws_bytes = F.fp4_quantize_workspace(self.batch, self.rows, self.cols, self.opts)
        self.ws = torch.empty((max(self.ws_bytes, 16),), dtype=torch.uint8, device=dev)
        self.dt = F.FP4_BF16 if x.dtype == torch.bfloat16 else F.FP4_F32
        self.nv = fmt == F.FP4_NVFP4
        self.fmt = fmt
        self.flags = flags
        self.stream = torch.cuda.current_stream().cuda_stream
        self.lib = F.lib()
        self.opts_ref = ctypes.byref(self.opts)

    def __call__(self, i):
        x = self.xs[i % len(self.xs)]
        st = self.lib.fp4_quantize(x.data_ptr(), self.dt, self.batch, self.rows, self.cols, self.cols,
                                   self.rows * self.cols, self.opts_ref, self.codes.data_ptr(), self.ldc,
                                   self.R * self.ldc, self.scales_buf.data_ptr(), self.lds,
                                   self.R * self.lds, self.ts.data_ptr(), self.ws.data_ptr(),
                                   self.ws_bytes, self.stream)
        if st != 0:
            raise RuntimeError(f"fp4_quantize: {self.F.fp4_status_str(st)}")

    def bytes(self):
        return quant_bytes(self.batch * self.rows * self.cols, 2 if self.dt == self.F.FP4_BF16 else 4, self.blk,
                           self.nv, self.batch)

    def quantized(self):
        return self.F.Quantized(self.fmt, self.codes, self.scales, self.ts if self.nv else None)

    def kernel(self):
        """The quantizer instantiation fp4_quantize launches for this call, by
        the dispatch of csrc/quantize.hip (quant_rows_kernel or, transposed,
        quant_cols_kernel<input, NVFP4, scale selection, 2D, SR, RHT>), after
        the amax pre-pass (amax_kernel<input, plain / RHT rows / RHT columns>,
        then amax_finalize_kernel) when NVFP4 runs without a supplied amax;
        the kernels of one call are joined by '+'. The label only keys the
        kernels in profiles."""
        F, f = self.F, self.flags
        b = lambda v: "true" if v else "false"
        if not self.nv:
            sel = 1 if f & F.FP4_FOUR_OVER_SIX else 0
        elif f & F.FP4_TENSOR_SCALE:
            sel = 3
        elif f & F.FP4_SCALE_SEARCH:
            sel = 2
        else:
            sel = 1 if f & F.FP4_FOUR_OVER_SIX else 0
        b2d = self.nv and sel != 3 and bool(f & F.FP4_BLOCK2D)
        name = "quant_cols_kernel" if f & F.FP4_TRANSPOSE else "quant_rows_kernel"
        tin = "unsigned short" if self.dt == F.FP4_BF16 else "float"
        k = (f"{name}<{tin}, {b(self.nv)}, {sel}, {b(b2d)}, {b(f & F.FP4_STOCHASTIC)}, "
             f"{b(f & F.FP4_HADAMARD)}>")
        if not (self.nv and self.amax is None):
            return k
        mode = 0 if not f & F.FP4_HADAMARD else (2 if f & F.FP4_TRANSPOSE else 1)
        return f"amax_kernel<{tin}, {mode}>+amax_finalize_kernel+{k}"


def gemm_kernel_label(nv, G, M, N, K, out_kind, routed=False):
    """The gemm_fp4_kernel instantiation that fp4_gemm launches, by the tile
    rule of launch_gemm in csrc/gemm.hip: 256-wide tiles when they still give
    every compute unit a tile (for NVFP4 only from K = 1024 and with a plain
    output), else 128-wide. The label only keys the kernel in profiles."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mt = (M + 255) // 256 * (1 if routed else G)
    wide = (N + 255) // 256 * mt >= cus
    bn = 256 if wide and out_kind < 2 and (not nv or K >= 1024) else 128
    b = lambda v: "true" if v else "false"
    return f"gemm_fp4_kernel<{b(nv)}, {bn}, 4, {out_kind}, {b(routed)}>"


class GemmCall:
    def __init__(self, F, qa, qb, out_dtype=torch.bfloat16):
        self.F, self.lib = F, F.lib()
        self.a, self.b = qa.quantized(), qb.quantized()
        self.G, self.M, half = self.a.codes.shape
        self.N = self.b.codes.shape[1]
        self.K = half * 2
        self.c = torch.empty((self.G, self.M, self.N), dtype=out_dtype, device=self.a.codes.device)
        self.ct = F.FP4_BF16 if out_dtype == torch.bfloat16 else F.FP4_F32
        self.stream = torch.cuda.current_stream().cuda_stream
        a, b = self.a, self.b
        self.args = (a.fmt, self.G, self.M, self.N, self.K, a.codes.data_ptr(), a.codes.stride(1),
                     a.codes.stride(0), a.scales.data_ptr(), a.scales.stride(1), a.scales.stride(0),
                     a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                     b.codes.data_ptr(), b.codes.stride(1), b.codes.stride(0), b.scales.data_ptr(),
                     b.scales.stride(1), b.scales.stride(0),
                     b.tensor_scale.data_ptr() if b.tensor_scale is not None else None,
                     self.c.data_ptr(), self.ct, self.N, self.M * self.N)

    def __call__(self, i):
        st = self.lib.fp4_gemm(*self.args, self.stream)
        if st != 0:
            raise RuntimeError(f"fp4_gemm: {self.F.fp4_status_str(st)}")

    def flops(self):
        return 2.0 * self.G * self.M * self.N * self.K

    def kernel(self):
        return gemm_kernel_label(self.a.fmt == self.F.FP4_NVFP4, self.G, self.M, self.N, self.K,
                                 1 if self.ct == self.F.FP4_BF16 else 0)


class GemmQuantizeOutputCall:
    """fp4_gemm_quantize_output: the product quantized in the epilogue to
    NVFP4 4/6 with a supplied amax (taken once, untimed, from the unfused
    product: the amax a previous step would hand over)."""

    def __init__(self, F, qa, qb, amax):
        self.F, self.lib = F, F.lib()
        a, b = qa.quantized(), qb.quantized()
        self.G, self.M, half = a.codes.shape
        self.N = b.codes.shape[1]
        self.K = half * 2
        dev = a.codes.device
        self.amax = amax.to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
        self.opts = F.make_opts(F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX, 0, 0, 0, self.amax.data_ptr())
        self.codes = torch.empty((self.G, self.M, self.N // 2), dtype=torch.uint8, device=dev)
        self.lds = F.scale_pitch(self.N // 16)
        self.scales = torch.empty((self.G, self.M, self.lds), dtype=torch.uint8, device=dev)
        self.ts = torch.empty((self.G,), dtype=torch.float32, device=dev)
        self.args = (a.fmt, self.G, self.M, self.N, self.K, a.codes.data_ptr(), a.codes.stride(1),
                     a.codes.stride(0), a.scales.data_ptr(), a.scales.stride(1), a.scales.stride(0),
                     a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                     b.codes.data_ptr(), b.codes.stride(1), b.codes.stride(0), b.scales.data_ptr(),
                     b.scales.stride(1), b.scales.stride(0),
                     b.tensor_scale.data_ptr() if b.tensor_scale is not None else None,
                     ctypes.byref(self.opts), self.codes.data_ptr(), self.N // 2, self.M * (self.N // 2),
                     self.scales.data_ptr(), self.lds, self.M * self.lds, self.ts.data_ptr())
        self.stream = torch.cuda.current_stream().cuda_stream

    def __call__(self, i):
        st = self.lib.fp4_gemm_quantize_output(*self.args, self.stream)
        if st != 0:
            raise RuntimeError(f"fp4_gemm_quantize_output: {self.F.fp4_status_str(st)}")

    def flops(self):
        return 2.0 * self.G * self.M * self.N * self.K


class GroupedGemmCall:
    """fp4_gemm_grouped over A [M, K] (one quantized tensor) and B [G, N, K],
    group rows from device offsets."""

    def __init__(self, F, qa, qb, offsets, out_dtype=torch.bfloat16):
        self.F, self.lib = F, F.lib()
        a, b = qa.quantized(), qb.quantized()
        _, self.M, half = a.codes.shape
        self.G, self.N = b.codes.shape[0], b.codes.shape[1]
        self.K = half * 2
        self.offsets = offsets.to(device=a.codes.device, dtype=torch.int32)
        self.c = torch.empty((self.M, self.N), dtype=out_dtype, device=a.codes.device)
        ct = F.FP4_BF16 if out_dtype == torch.bfloat16 else F.FP4_F32
        self.args = (a.fmt, self.G, self.offsets.data_ptr(), self.M, self.N, self.K, a.codes.data_ptr(),
                     a.codes.stride(1), a.scales.data_ptr(), a.scales.stride(1),
                     a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                     b.codes.data_ptr(), b.codes.stride(1), b.codes.stride(0), b.scales.data_ptr(),
                     b.scales.stride(1), b.scales.stride(0),
                     b.tensor_scale.data_ptr() if b.tensor_scale is not None else None,
                     self.c.data_ptr(), ct, self.N)
        self.stream = torch.cuda.current_stream().cuda_stream

    def __call__(self, i):
        st = self.lib.fp4_gemm_grouped(*self.args, self.stream)
        if st != 0:
            raise RuntimeError(f"fp4_gemm_grouped: {self.F.fp4_status_str(st)}")

    def flops(self):
        return 2.0 * self.M * self.N * self.K


def n_sets(bytes_per_set):
    return max(2, -(-ROTATE_BYTES // max(bytes_per_set, 1)))


def copies(t, n):
    return [t] + [t.clone() for _ in range(n - 1)]




# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass
class QuantSample:
    """A CPU-baseline sample of one quantize op: the oracle quantizes
    `units` rows (axis 0) or columns (axis 1: a transposed quantize, whose
    output rows are the source columns) of x; the time scales by
    full_units / units to the whole op, batch items included."""
    name: str
    x: np.ndarray           # bf16 bit patterns (uint16) or float32
    fmt: int
    flags: int
    axis: int
    full_units: int
    bytes_full: int
    one: int                # units timed on one core
    all: int                # units timed on all cores (split over processes)
    signs: int = 0
    seed: int = 0
    offset: int = 0
    step: int = 16          # units come in multiples of this (2D tiles, lane pairs)


@dataclass
class GemmSample:
    """A CPU-baseline sample of one GEMM: the oracle's operands of m_s rows
    of A and n_s rows of B (quantized untimed), then its dequantize (timed,
    scaled by (M + N) / (m_s + n_s)) and its float64 matmul (timed, scaled
    by M N / (m_s n_s)), times `groups`."""
    name: str
    a: np.ndarray           # A rows [>= m_s, K] (bf16 bits)
    b: np.ndarray           # B as [N, K] rows, or [K, N] with b_transposed
    b_transposed: bool
    fmt: int
    fa: int
    fb: int
    M: int
    N: int
    K: int
    groups: int
    one: tuple
    all: tuple
    signs: int = 0


@dataclass
class Workload:
    ops: list
    cfg: dict
    dtype: str
    cpu: list = field(default_factory=list)      # CPU-baseline samples
    probes: list = field(default_factory=list)   # ops timed on their own, outside the step


def sylvester16(device):
    h = torch.ones(1, 1)
    for _ in range(4):
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h.to(device)


def probe_amax(x, hadamard=False, signs=0, along_columns=False):
    """The tensor amax the quantizer's pre-pass finds (after the random
    Hadamard transform along the block direction, if on), computed with
    torch for the kernel-only timing of an NVFP4 quantize (the value only
    sets the tensor scale; any positive amax does the same work)."""
    xf = x.float()
    if not hadamard:
        return xf.abs().amax().reshape(1)
    if along_columns:
        xf = xf.t()
    d = torch.tensor([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)], device=x.device)
    m = (sylvester16(x.device) * d[None, :]) / 4.0
    best = torch.zeros((), device=x.device)
    rows = xf.shape[0]
    for r in range(0, rows, 2048):
        v = xf[r:r + 2048].contiguous().reshape(-1, 16) @ m.t()
        best = torch.maximum(best, v.abs().amax())
    return best.reshape(1)


def bits(t):
    """bf16 device/host tensor -> numpy uint16 bit patterns (host)."""
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def kernel_only(F, name, xs, fmt, flags, amax, signs=0, seed=0, offset=0):
    q = QuantCall(F, xs, fmt, flags, signs=signs, seed=seed, offset=offset, amax=amax)
    return Op(name + " (kernel only, amax supplied)", q.kernel(), "hbm", q.bytes(), PEAK_HBM_GBS, q, "GB/s")


def wl_w4a4_linear(F, inputs):
    d = inputs.w4a4_linear(device="cuda")
    n = n_sets(d["a"].numel() * 2 + d["w"].numel() * 2)
    fos = F.FP4_FOUR_OVER_SIX
    xa, xw = copies(d["a"], n), copies(d["w"], n)
    qa = QuantCall(F, xa, F.FP4_NVFP4, fos)
    qw = QuantCall(F, xw, F.FP4_NVFP4, fos)
    gm = GemmCall(F, qa, qw, torch.bfloat16)
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", qa.kernel(), "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", qw.kernel(), "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", gm.kernel(), "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s")]
    probes = [kernel_only(F, "quantize A nvfp4 4/6", xa, F.FP4_NVFP4, fos, probe_amax(d["a"])),
              kernel_only(F, "quantize W nvfp4 4/6", xw, F.FP4_NVFP4, fos, probe_amax(d["w"]))]
    cfg = {"workload": "w4a4_linear_nvfp4_four_over_six", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "bf16", "input_sets_rotated": n}
    a, w = bits(d["a"]), bits(d["w"])
    cpu = [QuantSample("quantize A nvfp4 4/6", a, F.FP4_NVFP4, fos, 0, 2048, qa.bytes(), 512, 2048),
           QuantSample("quantize W nvfp4 4/6", w, F.FP4_NVFP4, fos, 0, 4096, qw.bytes(), 512, 4096),
           GemmSample("gemm nvfp4", a, w, False, F.FP4_NVFP4, fos, fos, 2048, 4096, 4096, 1, (128, 1024), (512, 4096))]
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", cpu, probes)


def wl_moe(F, inputs):
    d = inputs.moe_mxfp4(device="cuda")
    n = n_sets(d["w"].numel() * 2 + d["x"].numel() * 2)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_MXFP4, F.FP4_TRANSPOSE)
    qx = QuantCall(F, copies(d["x"], n), F.FP4_MXFP4, 0)
    gm = GemmCall(F, qx, qw, torch.bfloat16)
    ops = [Op("quantize W^T mxfp4 32x[2880x5760]", qw.kernel(), "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("quantize X mxfp4 32x[512x2880]", qx.kernel(), "hbm", qx.bytes(),
              PEAK_HBM_GBS, qx, "GB/s"),
           Op("grouped gemm mxfp4 (scaled FP4 MFMA)", gm.kernel(), "mfma",
              gm.flops(), PEAK_TFLOPS["fp4"], gm, "TFLOP/s")]
    cfg = {"workload": "moe_mxfp4_grouped_32x512x5760x2880", "experts": 32, "M": 512, "N": 5760, "K": 2880,
           "output": "bf16", "input_sets_rotated": n}
    # four experts' weights side by side as [K, 4 N] (their transposed
    # quantize is the four experts' stacked), their tokens as [4 * 512, K]
    w4 = bits(torch.cat([d["w"][e] for e in range(4)], dim=1))
    x4 = bits(d["x"][:4].reshape(4 * 512, 2880))
    cpu = [QuantSample("quantize W^T mxfp4", w4, F.FP4_MXFP4, F.FP4_TRANSPOSE, 1, 32 * 5760, qw.bytes(), 5760,
                       4 * 5760),
           QuantSample("quantize X mxfp4", x4, F.FP4_MXFP4, 0, 0, 32 * 512, qx.bytes(), 512, 2048),
           GemmSample("grouped gemm mxfp4", x4[:512], w4[:, :5760], True, F.FP4_MXFP4, 0, F.FP4_TRANSPOSE, 512, 5760,
                      2880, 32, (512, 2880), (512, 5760))]
    return Workload(ops, cfg, "fp4 e2m1 codes (mxfp4); fp4 MFMA, f32 accumulate", cpu)


def wl_training(F, inputs):
    d = inputs.training(device="cuda")
    n = n_sets(d["w"].numel() * 4)
    # W and W^T read their own copies: a second read of the same tensor right
    # after the first would be served from the 256 MB Infinity Cache
    ws, ws2, gs = copies(d["w"], n), copies(d["w"], n), copies(d["grad"], n)
    f = F.FP4_FOUR_OVER_SIX | F.FP4_BLOCK2D
    fg = F.FP4_FOUR_OVER_SIX | F.FP4_STOCHASTIC
    q1 = QuantCall(F, ws, F.FP4_NVFP4, f)
    q2 = QuantCall(F, ws2, F.FP4_NVFP4, f | F.FP4_TRANSPOSE)
    q3 = QuantCall(F, gs, F.FP4_NVFP4, fg, seed=d["sr_seed"])
    ops = [Op("quantize W nvfp4 2D 4/6", q1.kernel(), "hbm", q1.bytes(), PEAK_HBM_GBS, q1, "GB/s", lane=1),
           Op("quantize W^T nvfp4 2D 4/6", q2.kernel(), "hbm", q2.bytes(), PEAK_HBM_GBS, q2, "GB/s", lane=2),
           Op("quantize G nvfp4 4/6 stochastic", q3.kernel(), "hbm", q3.bytes(),
              PEAK_HBM_GBS, q3, "GB/s", lane=3)]
    aw, ag = probe_amax(d["w"]), probe_amax(d["grad"])
    probes = [kernel_only(F, "quantize W nvfp4 2D 4/6", ws, F.FP4_NVFP4, f, aw),
              kernel_only(F, "quantize W^T nvfp4 2D 4/6", ws2, F.FP4_NVFP4, f | F.FP4_TRANSPOSE,
                          aw),
              kernel_only(F, "quantize G nvfp4 4/6 stochastic", gs, F.FP4_NVFP4, fg, ag,
                          seed=d["sr_seed"])]
    cfg = {"workload": "training_quantize_nvfp4_8192x8192", "shape": [8192, 8192], "input_sets_rotated": n}
    w, g = bits(d["w"][:, :2048].contiguous()), bits(d["grad"][:1024])
    wrows = bits(d["w"][:1024])
    cpu = [QuantSample("quantize W nvfp4 2D 4/6", wrows, F.FP4_NVFP4, f, 0, 8192, q1.bytes(), 128, 1024),
           QuantSample("quantize W^T nvfp4 2D 4/6", w, F.FP4_NVFP4, f | F.FP4_TRANSPOSE, 1, 8192, q2.bytes(), 128,
                       2048),
           QuantSample("quantize G nvfp4 4/6 stochastic", g, F.FP4_NVFP4, fg, 0, 8192, q3.bytes(), 128, 1024,
                       seed=d["sr_seed"])]
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4), f32 scale arithmetic", cpu, probes)


def wl_rht(F, inputs):
    d = inputs.rht_activation(device="cuda")
    n = n_sets(d["x"].numel() * 2 + d["w"].numel() * 2)
    f = F.FP4_FOUR_OVER_SIX | F.FP4_HADAMARD
    xs, wsets = copies(d["x"], n), copies(d["w"], n)
    qx = QuantCall(F, xs, F.FP4_NVFP4, f, signs=d["signs"])
    qw = QuantCall(F, wsets, F.FP4_NVFP4, f | F.FP4_TRANSPOSE, signs=d["signs"])
    gm = GemmCall(F, qx, qw, torch.bfloat16)
    ops = [Op("quantize X nvfp4 4/6 RHT", qx.kernel(), "hbm", qx.bytes(), PEAK_HBM_GBS, qx, "GB/s", lane=1),
           Op("quantize W^T nvfp4 4/6 RHT", qw.kernel(), "hbm", qw.bytes(), PEAK_HBM_GBS, qw, "GB/s", lane=2),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", gm.kernel(), "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s")]
    probes = [kernel_only(F, "quantize X nvfp4 4/6 RHT", xs, F.FP4_NVFP4, f,
                          probe_amax(d["x"], True, d["signs"]), signs=d["signs"]),
              kernel_only(F, "quantize W^T nvfp4 4/6 RHT", wsets, F.FP4_NVFP4,
                          f | F.FP4_TRANSPOSE, probe_amax(d["w"], True, d["signs"], along_columns=True),
                          signs=d["signs"])]
    cfg = {"workload": "rht_activation_nvfp4_16384x12288x4096", "M": 16384, "N": 12288, "K": 4096,
           "activations": "16384x4096 bf16 N(0,1) + 0.5% Student-t(2)", "weight": "4096x12288 bf16 N(0,0.02) as [K, N]",
           "transform": "16-point random Hadamard, one sign mask for both operands", "output": "bf16",
           "input_sets_rotated": n}
    x, w = bits(d["x"][:8192]), bits(d["w"][:, :6144].contiguous())
    cpu = [QuantSample("quantize X nvfp4 4/6 RHT", x, F.FP4_NVFP4, f, 0, 16384, qx.bytes(), 2048, 8192,
                       signs=d["signs"]),
           QuantSample("quantize W^T nvfp4 4/6 RHT", w, F.FP4_NVFP4, f | F.FP4_TRANSPOSE, 1, 12288, qw.bytes(), 1536,
                       6144, signs=d["signs"]),
           GemmSample("gemm nvfp4", x, w, True, F.FP4_NVFP4, f, f | F.FP4_TRANSPOSE, 16384, 12288, 4096, 1,
                      (512, 1536), (2048, 6144), signs=d["signs"])]
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", cpu, probes)
def wl_training_backward(F, inputs):
    """Backward GEMMs of a quantized linear Y = X W^T (dgrad, wgrad), each with
    its operands' quantization: dX = Q(dY) Q(W^T)^T with the weight's 2D
    16x16 scales (the same scales as its forward quantization), and
    dW = Q(dY^T) Q(X^T)^T; gradients with stochastic rounding (a different
    Philox offset for each of the two quantizations of dY)."""
    d = inputs.training_backward(device="cuda")
    n = n_sets(d["w"].numel() * 2 + d["grad"].numel() * 2 + d["x"].numel() * 2)
    # the two quantizations of dY read separate copies (no cache-served re-read)
    gs, gs2, ws, xs = copies(d["grad"], n), copies(d["grad"], n), copies(d["w"], n), copies(d["x"], n)
    fos, sr, tr = F.FP4_FOUR_OVER_SIX, F.FP4_STOCHASTIC, F.FP4_TRANSPOSE
    qg = QuantCall(F, gs, F.FP4_NVFP4, fos | sr, seed=d["sr_seed"], offset=0)
    qwt = QuantCall(F, ws, F.FP4_NVFP4, fos | F.FP4_BLOCK2D | tr)
    gd = GemmCall(F, qg, qwt, torch.bfloat16)
    qgt = QuantCall(F, gs2, F.FP4_NVFP4, fos | sr | tr, seed=d["sr_seed"], offset=1 << 40)
    qxt = QuantCall(F, xs, F.FP4_NVFP4, fos | tr)
    gw = GemmCall(F, qgt, qxt, torch.bfloat16)
    ops = [Op("quantize dY nvfp4 4/6 stochastic", qg.kernel(), "hbm", qg.bytes(),
              PEAK_HBM_GBS, qg, "GB/s", lane=1),
           Op("quantize W^T nvfp4 2D 4/6", qwt.kernel(), "hbm", qwt.bytes(), PEAK_HBM_GBS, qwt, "GB/s", lane=2),
           Op("dgrad gemm nvfp4 dX = dY W", gd.kernel(), "mfma", gd.flops(),
              PEAK_TFLOPS["f16"], gd, "TFLOP/s"),
           Op("quantize dY^T nvfp4 4/6 stochastic", qgt.kernel(), "hbm", qgt.bytes(), PEAK_HBM_GBS, qgt,
              "GB/s", lane=1),
           Op("quantize X^T nvfp4 4/6", qxt.kernel(), "hbm", qxt.bytes(), PEAK_HBM_GBS, qxt, "GB/s", lane=2),
           Op("wgrad gemm nvfp4 dW = dY^T X", gw.kernel(), "mfma", gw.flops(),
              PEAK_TFLOPS["f16"], gw, "TFLOP/s")]
    cfg = {"workload": "training_backward_nvfp4_8192", "M": 8192, "N": 8192, "K": 8192,
           "gradient": "8192x8192 bf16 Laplace(0,1e-3)", "weight": "8192x8192 bf16 N(0,0.02)",
           "activations": "8192x8192 bf16 N(0,1)", "output": "bf16", "input_sets_rotated": n}
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate")


def wl_w4a4_fused(F, inputs):
    """The W4A4 linear layer handing NVFP4 4/6 activations to the next one:
    its GEMM quantizes C in the epilogue instead of storing bf16 C."""
    d = inputs.w4a4_linear(device="cuda")
    n = n_sets(d["a"].numel() * 2 + d["w"].numel() * 2)
    qa = QuantCall(F, copies(d["a"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    qa(0)
    qw(0)
    probe = GemmCall(F, qa, qw, torch.float32)
    probe(0)
    amax = probe.c.abs().amax().reshape(1)
    del probe
    gq = GemmQuantizeOutputCall(F, qa, qw, amax)
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", qa.kernel(), "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", qw.kernel(), "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4, output quantized to nvfp4 4/6 in the epilogue", "gemm_fp4_kernel<true, 128, 4, 3, false>",
              "mfma", gq.flops(), PEAK_TFLOPS["f16"], gq, "TFLOP/s")]
    cfg = {"workload": "w4a4_linear_nvfp4_fused_output_quantize", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "nvfp4 4/6 codes + scales, amax supplied", "input_sets_rotated": n}
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate")


def wl_w4a4_unfused_chain(F, inputs):
    """The same hand-over as w4a4_fused done the unfused way, for
    comparison: the GEMM stores bf16 C, then C is quantized to NVFP4 4/6
    with the same supplied amax."""
    d = inputs.w4a4_linear(device="cuda")
    n = n_sets(d["a"].numel() * 2 + d["w"].numel() * 2)
    qa = QuantCall(F, copies(d["a"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    qa(0)
    qw(0)
    gm = GemmCall(F, qa, qw, torch.bfloat16)
    gm(0)
    amax = gm.c.float().abs().amax().reshape(1)
    qc = QuantCall(F, [gm.c], F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX, amax=amax)
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", qa.kernel(), "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", qw.kernel(), "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", gm.kernel(), "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s"),
           Op("quantize C nvfp4 4/6 (amax supplied)", qc.kernel(), "hbm", qc.bytes(), PEAK_HBM_GBS, qc,
              "GB/s")]
    cfg = {"workload": "w4a4_linear_nvfp4_unfused_output_quantize", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "bf16 C, then nvfp4 4/6 codes + scales, amax supplied", "input_sets_rotated": n}
    return Workload(ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate")


def wl_scale_search(F, inputs):
    """The error-searched scale options on the training weight (8192^2 bf16):
    NVFP4 with the scale search over every E4M3 code between the 4 and 6
    candidates, 1D and 2D, and MXFP4 with the 4/6 exponent pair."""
    d = inputs.training(device="cuda")
    n = n_sets(d["w"].numel() * 2)
    # one set of copies per op, so no op reads what the previous one just read
    qs = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, F.FP4_SCALE_SEARCH)
    q2 = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, F.FP4_SCALE_SEARCH | F.FP4_BLOCK2D)
    qm = QuantCall(F, copies(d["w"], n), F.FP4_MXFP4, F.FP4_FOUR_OVER_SIX)
    ops = [Op("quantize W nvfp4 scale search (amax pre-pass + quantize)", qs.kernel(), "hbm",
              qs.bytes(), PEAK_HBM_GBS, qs, "GB/s", lane=1),
           Op("quantize W nvfp4 2D scale search (amax pre-pass + quantize)", q2.kernel(), "hbm",
              q2.bytes(), PEAK_HBM_GBS, q2, "GB/s", lane=2),
           Op("quantize W mxfp4 4/6 exponent pair", qm.kernel(), "hbm", qm.bytes(),
              PEAK_HBM_GBS, qm, "GB/s", lane=3)]
    cfg = {"workload": "scale_search_8192", "shape": [8192, 8192], "weight": "8192x8192 bf16 N(0,0.02)",
           "input_sets_rotated": n}
    return Workload(ops, cfg, "fp4 e2m1 codes, f32 scale arithmetic")


def wl_moe_routed(F, inputs):
    """MoE layer with router-decided rows per expert: 4096 tokens top-4 over
    32 experts (16384 rows, 60 to 1709 per expert), one MXFP4 quantize of the
    routed tokens, and the grouped GEMM reading the row offsets on the
    device."""
    d = inputs.moe_routed(device="cuda")
    n = n_sets(d["w"].numel() * 2 + d["x"].numel() * 2)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_MXFP4, F.FP4_TRANSPOSE)
    qx = QuantCall(F, copies(d["x"], n), F.FP4_MXFP4, 0)
    gm = GroupedGemmCall(F, qx, qw, d["offsets"], torch.bfloat16)
    ops = [Op("quantize W^T mxfp4 32x[2880x5760]", qw.kernel(), "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("quantize routed X mxfp4 [16384x2880]", qx.kernel(), "hbm", qx.bytes(), PEAK_HBM_GBS, qx,
              "GB/s"),
           Op("grouped gemm mxfp4, router row counts", "gemm_fp4_kernel<false, 256, 4, 1, true>", "mfma",
              gm.flops(), PEAK_TFLOPS["fp4"], gm, "TFLOP/s")]
    cfg = {"workload": "moe_mxfp4_routed", "experts": 32, "tokens": 4096, "top_k": 4, "rows": int(d["offsets"][-1]),
           "rows_per_expert": [int(v) for v in d["counts"]], "N": 5760, "K": 2880, "output": "bf16",
           "input_sets_rotated": n}
    return Workload(ops, cfg, "fp4 e2m1 codes (mxfp4); fp4 MFMA, f32 accumulate")



WORKLOADS = {"rht": wl_rht, "moe": wl_moe, "training": wl_training, "w4a4_linear": wl_w4a4_linear,
             "training_backward": wl_training_backward, "moe_routed": wl_moe_routed, "w4a4_fused": wl_w4a4_fused,
             "w4a4_unfused_chain": wl_w4a4_unfused_chain, "scale_search": wl_scale_search}
# the configurations the default line carries beside the headline step
EXTRA_WORKLOADS = ("moe", "training", "w4a4_linear")
# the ones given a CPU baseline in the default line: every configuration it carries
CPU_WORKLOADS = ("rht", "moe", "training", "w4a4_linear")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on one core and on all host cores
# ---------------------------------------------------------------------------
def host_cores():
    """Cores this process may run on, at most 16 (the machine's CPU share per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def split(units, parts, step):
    """units (a multiple of step) into `parts` ranges of whole steps."""
    chunks = units // step
    parts = max(1, min(parts, chunks))
    bounds = [step * (chunks * i // parts) for i in range(parts + 1)]
    return [(bounds[i], bounds[i + 1]) for i in range(parts) if bounds[i + 1] > bounds[i]]


def cpu_quantize(s: QuantSample, units, workers, tmp):
    """Seconds the oracle takes to quantize `units` of the sample, the units
    split over `workers` concurrent processes (span of their oracle calls)."""
    path = Path(tmp) / f"{abs(hash(s.name))}.npy"
    if not path.exists():
        np.save(path, s.x)
    procs = []
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    for i, (a, b) in enumerate(split(units, workers, s.step)):
        task = Path(tmp) / f"task_{i}.json"
        task.write_text(json.dumps({"input": str(path), "fmt": s.fmt, "flags": s.flags, "signs": s.signs,
                                    "seed": s.seed, "offset": s.offset, "axis": s.axis, "start": a, "stop": b}))
        procs.append(subprocess.Popen([sys.executable, str(ROOT / "oracle" / "cpu_worker.py"), str(task)],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env))
    spans = []
    for p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"cpu_worker failed: {err[-2000:]}")
        spans.append(json.loads(out.strip().splitlines()[-1]))
    return max(t["t1"] for t in spans) - min(t["t0"] for t in spans), len(procs)


def cpu_gemm(g: GemmSample, m_s, n_s, threads):
    """Oracle dequantize of m_s rows of A and n_s rows of B, then the
    reference matmul (float64, the BLAS limited to `threads`); seconds
    scaled to the whole GEMM."""
    from threadpoolctl import threadpool_limits

    from oracle import oracle as O
    qa = O.quantize(np.ascontiguousarray(g.a[:m_s]), g.fmt, flags=g.fa, rht_signs=g.signs)
    bsrc = np.ascontiguousarray(g.b[:, :n_s] if g.b_transposed else g.b[:n_s])
    qb = O.quantize(bsrc, g.fmt, flags=g.fb, rht_signs=g.signs)
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        da = O.dequantize(g.fmt, qa["codes"], qa["scales"], qa["tensor_scale"])
        db = O.dequantize(g.fmt, qb["codes"], qb["scales"], qb["tensor_scale"])
        t1 = time.perf_counter()
        O.gemm_reference(da, db)
        t2 = time.perf_counter()
    full = g.groups * ((t1 - t0) * (g.M + g.N) / (m_s + n_s) + (t2 - t1) * (g.M * g.N) / (m_s * n_s))
    return full, t2 - t0


def cpu_baseline(wl: Workload, roof_s):
    """Both legs of the CPU baseline of a workload's step."""
    from oracle import oracle as O
    O.lib()  # built once here, before any worker loads it
    cores = host_cores()
    legs = {}
    with tempfile.TemporaryDirectory(prefix="fp4_cpu_") as tmp:
        for leg, workers in (("one_core", 1), ("all_cores", cores)):
            ops, total, measured, used = [], 0.0, 0.0, 1
            for s in wl.cpu:
                if isinstance(s, QuantSample):
                    units = s.one if workers == 1 else s.all
                    t, n = cpu_quantize(s, units, workers, tmp)
                    full = t * s.full_units / units
                    used = max(used, n)
                    ops.append({"op": s.name, "sample": f"{units} of {s.full_units} "
                                f"{'source columns' if s.axis else 'rows'}", "seconds": round(t, 3),
                                "full_seconds": round(full, 3), "GBps": round(s.bytes_full / full / 1e9, 5)})
                else:
                    m_s, n_s = s.one if workers == 1 else s.all
                    full, t = cpu_gemm(s, m_s, n_s, workers)
                    used = max(used, workers)
                    flops = 2.0 * s.groups * s.M * s.N * s.K
                    ops.append({"op": s.name, "sample": f"{m_s} x {n_s} of {s.M} x {s.N} outputs"
                                f"{f' (one of {s.groups} groups)' if s.groups > 1 else ''}, K {s.K}",
                                "seconds": round(t, 3), "full_seconds": round(full, 3),
                                "TFLOPs": round(flops / full / 1e12, 6)})
                total += full
                measured += t
            legs[leg] = {"value": round(100.0 * roof_s / total, 6), "cores": used,
                         "step_seconds": round(total, 3), "measured_seconds": round(measured, 3), "ops": ops}
    a = legs["all_cores"]
    return {"value": a["value"], "unit": "% of roofline (step)", "cores": a["cores"], "kind": "oracle",
            "sample": "; ".join(f"{o['op']}: {o['sample']}" for o in a["ops"]) + "; each scaled to the full op",
            "cpu_model": cpu_model(), "step_seconds": a["step_seconds"], "measured_seconds": a["measured_seconds"],
            "ops": a["ops"], "one_core": legs["one_core"]}


# ---------------------------------------------------------------------------
# the worked example: codes, scales and MAE in every mode
# ---------------------------------------------------------------------------
def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def worked_example_record(F, inputs):
    """The 4096-value example ("FP4" glossary, "Como funciona FP4") in the
    whole-tensor, MXFP4, NVFP4 and NVFP4 four-over-six modes, on the GPU:
    digests of the codes, scale bytes and tensor scale, and the MAE of the
    dequantized tensor; beside them, as this configuration's CPU baseline,
    the oracle's, and the page's printed MAE of its float-scale modes."""
    from oracle import oracle as O
    x = inputs.worked_example().reshape(1, 4096)
    xd = x.cuda()
    modes = {"whole_tensor": (F.FP4_NVFP4, F.FP4_TENSOR_SCALE), "mxfp4": (F.FP4_MXFP4, 0),
             "nvfp4": (F.FP4_NVFP4, 0), "nvfp4_four_over_six": (F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)}
    out = {"workload": "worked_example_4096", "input": "4096 fp32 N(0,1), seed 0, every 512th x20", "modes": {}}
    xn = x.numpy().astype(np.float64)
    for name, (fmt, fl) in modes.items():
        q = F.quantize(xd, fmt, four_over_six=bool(fl & F.FP4_FOUR_OVER_SIX),
                       tensor_scale=bool(fl & F.FP4_TENSOR_SCALE))
        deq = F.dequantize(q).cpu().numpy().astype(np.float64)
        codes, scales = q.codes.cpu().numpy(), q.scales.cpu().numpy()
        ts = q.tensor_scale.cpu().numpy() if q.tensor_scale is not None else np.zeros(0, np.float32)
        gpu = {"codes_sha256": sha(codes), "scales_sha256": sha(scales), "tensor_scale": [float(v) for v in ts],
               "mae": float(np.abs(deq - xn).mean())}
        r = O.quantize(x.numpy(), fmt, flags=fl)
        od = O.dequantize(fmt, r["codes"], r["scales"], r["tensor_scale"]).astype(np.float64)
        ots = np.array([r["tensor_scale"]], np.float32) if r["tensor_scale"] is not None else np.zeros(0, np.float32)
        orc = {"codes_sha256": sha(r["codes"]), "scales_sha256": sha(r["scales"]),
               "tensor_scale": [float(v) for v in ots], "mae": float(np.abs(od - xn).mean())}
        out["modes"][name] = {"gpu": gpu, "oracle": orc,
                              "bit_exact": bool(np.array_equal(codes, r["codes"]) and np.array_equal(scales, r["scales"])
                                                and np.array_equal(ts.view(np.uint32), ots.view(np.uint32)))}
    gold = json.loads((ROOT / "tests" / "golden" / "worked_example.json").read_text())
    out["page_printed_mae_float_scale"] = {f"block_{k}": v for k, v in gold["mae"].items()}
    out["oracle_float_scale_mae"] = {f"block_{b}": float(np.abs(O.float_scale_dequant(x.numpy()[0], b) - xn[0]).mean())
                                     for b in (4096, 32, 16)}
    return out


# ---------------------------------------------------------------------------
KERNEL_SOURCES = {  # device sources each kernel family is built from
    "gemm": ["gemm.hip", "fp4_device.h", "launch.h"],
    "quant": ["quantize.hip", "quant_common.h", "fp4_device.h", "launch.h"],
    "dequant": ["dequantize.hip", "fp4_device.h", "launch.h"],
}


def own_kernel(label):
    """True for a kernel built from this library's device sources."""
    return label.split("<")[0] in ("amax_kernel", "amax_finalize_kernel", "quant_rows_kernel", "quant_cols_kernel",
                                   "gemm_fp4_kernel", "dequant_kernel")


def kernel_family(label):
    if label.startswith("gemm"):
        return "gemm"
    if label.startswith("dequant"):
        return "dequant"
    return "quant"


def source_digest(label=None):
    """Digest of the device sources a kernel is built from (all device
    sources when label is None): HBM counters taken on other sources are
    not reported."""
    csrc = ROOT / "block_scaled_fp4_amax_amd" / "csrc"
    names = sorted({n for v in KERNEL_SOURCES.values() for n in v}) if label is None else \
        KERNEL_SOURCES[kernel_family(label)]
    h = hashlib.sha256()
    for n in names:
        h.update(n.encode())
        h.update((csrc / n).read_bytes())
    return h.hexdigest()[:16]


def kernel_label(rocprof_name):
    """'void fp4impl::gemm_fp4_kernel<true, 128, 4, 1, false>(fp4impl::GemmArgs)'
    -> 'gemm_fp4_kernel<true, 128, 4, 1, false>'"""
    n = rocprof_name.split("(")[0]
    n = n[len("void "):] if n.startswith("void ") else n
    return n.split("::")[-1] if "<" not in n else n[n.rfind("::", 0, n.index("<")) + 2:]


def traffic_for(op_kernel, workload, table=None):
    """HBM bytes per launch of one op, from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None. An op
    of several kernels ('a+b+c') sums its kernels' entries. The counters are
    kept per kernel instantiation, averaged over its dispatches in the
    workload (ops of different sizes can share one), so a figure is only
    reported where those dispatches read nearly the same bytes (the spreads
    of the op's kernels add up to under 5 % of its total): the averages then
    are this op's own figures. table: the summary's contents (default: read
    from profiles/hbm_traffic.json)."""
    t = table
    if t is None:
        p = ROOT / "profiles" / "hbm_traffic.json"
        if not p.exists():
            return None
        try:
            t = json.loads(p.read_text())
        except ValueError:
            return None
    total = spread = 0
    for k in op_kernel.split("+"):
        e = t.get("workloads", {}).get(workload, {}).get(k)
        if not e or e.get("source_digest") != source_digest(k):
            return None
        total += e["bytes_per_launch"]
        spread += e.get("fetch_spread_bytes", total)
    if spread > 0.05 * total:
        return None
    return total


def read_pmc(dirpath, counter):
    """{kernel label: [value per dispatch]} from a rocprofv3 --pmc csv tree."""
    import csv
    out = {}
    for f in Path(dirpath).rglob("*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.setdefault(kernel_label(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def ingest_pmc(base, copy_bytes, commands):
    """Turn FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into HBM bytes per
    launch, each counter scaled by what it reads for a plain device copy of
    copy_bytes. Layout: base/<workload>/{fetch,write}, base/copy/{fetch,write}."""
    base = Path(base)
    cf = read_pmc(base / "copy" / "fetch", "FETCH_SIZE")
    cw = read_pmc(base / "copy" / "write", "WRITE_SIZE")
    ck = [k for k in cf if "copy" in k.lower()]
    if not ck:
        raise SystemExit("no copy kernel in the calibration run")
    fetch_kib = float(np.median(cf[ck[0]]))
    write_kib = float(np.median(cw[ck[0]]))
    f_fetch, f_write = copy_bytes / (fetch_kib * 1024.0), copy_bytes / (write_kib * 1024.0)
    out = {"calibration": {"copy_kernel": ck[0], "copy_bytes": copy_bytes, "fetch_kib": fetch_kib,
                           "write_kib": write_kib, "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
           "commands": commands, "workloads": {}}
    for wdir in sorted(p for p in base.iterdir() if p.is_dir() and p.name != "copy"):
        fe, wr = read_pmc(wdir / "fetch", "FETCH_SIZE"), read_pmc(wdir / "write", "WRITE_SIZE")
        ent = {}
        for k in fe:
            if k not in wr or not own_kernel(k):  # this library's kernels only
                continue
            fb = float(np.mean(fe[k])) * 1024.0 * f_fetch
            wb = float(np.mean(wr[k])) * 1024.0 * f_write
            ent[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                      "dispatches": len(fe[k]),
                      "fetch_spread_bytes": round((max(fe[k]) - min(fe[k])) * 1024.0 * f_fetch),
                      "source_digest": source_digest(k)}
        out["workloads"][wdir.name] = ent
    dst = ROOT / "profiles" / "hbm_traffic.json"
    dst.parent.mkdir(exist_ok=True)
    dst.write_text(json.dumps(out, indent=1) + "\n")
    print(f"wrote {dst}")


def calibrate_copy(nbytes, reps=5):
    """A plain device-to-device copy of nbytes, for scaling HBM counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)


def graph_step_ms(ops, steps, warmup):
    """Average step time with each step replayed as one captured HIP graph:
    the step's ops are captured once per input set (the ops read rotating
    copies, so each graph holds its own set's pointers) and the graphs are
    replayed round-robin. Every replay runs every kernel of the step; ops on
    side lanes (independent quantizations) run concurrently in the graph."""
    n = 1 + max(len(getattr(op.launch, "xs", [0])) for op in ops)
    cap = torch.cuda.Stream()
    sides = {op.lane: torch.cuda.Stream() for op in ops if op.lane > 0}
    saved = [op.launch.stream for op in ops]
    graphs = []
    try:
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                main = torch.cuda.current_stream()
                forked = set()
                for op in ops:
                    if op.lane > 0:
                        st = sides[op.lane]
                        if op.lane not in forked:
                            st.wait_stream(main)
                            forked.add(op.lane)
                        op.launch.stream = st.cuda_stream
                    else:
                        for k in forked:
                            main.wait_stream(sides[k])
                        forked.clear()
                        op.launch.stream = main.cuda_stream
                    op.launch(i)
                for k in forked:
                    main.wait_stream(sides[k])
            graphs.append(g)
    finally:
        for op, st in zip(ops, saved):
            op.launch.stream = st
    for k in range(warmup):
        graphs[k % n].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(steps):
        graphs[k % n].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps




def time_ops(ops, steps, warmup):
    """Eager timing. Each op alone: `steps` back-to-back launches (rotating
    input sets) between two HIP events on its stream, so that the queue stays
    ahead of the device and host launch latency does not enter an op's time;
    then the whole eager step (every op in order, `steps` times). Returns the
    per-op average durations (ms, one value per op) and the eager step (ms)."""
    torch.cuda.synchronize()
    for i in range(warmup):
        for op in ops:
            op.launch(i)
    torch.cuda.synchronize()
    per_op = []
    for op in ops:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            op.launch(i)
        e1.record()
        torch.cuda.synchronize()
        per_op.append([e0.elapsed_time(e1) / steps])
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(steps):
        for op in ops:
            op.launch(i)
    t_end.record()
    torch.cuda.synchronize()
    return per_op, t_start.elapsed_time(t_end) / steps


def op_record(op, durations, workload):
    avg_ms = float(np.mean(durations))
    achieved = op.work / (avg_ms * 1e-3) / (1e9 if op.unit == "GB/s" else 1e12)
    return {"op": op.name, "kernel": op.kernel, "bound": op.bound, "avg_ms": round(avg_ms, 5),
            "achieved": round(achieved, 2), "peak": op.peak, "unit": op.unit, "frac": round(achieved / op.peak, 4),
            "work_per_launch": op.work, "traffic": traffic_for(op.kernel, workload)}


def run(workload, steps, warmup, with_cpu):
    import block_scaled_fp4_amax_amd as F
    from block_scaled_fp4_amax_amd import inputs
    F.lib()
    torch.manual_seed(0)
    wl = WORKLOADS[workload](F, inputs)
    per_op, ms_step_eager = time_ops(wl.ops, steps, warmup)
    ms_step_graph = graph_step_ms(wl.ops, steps, warmup)
    # the step runs every op either way; the faster of the two launch forms
    # is the step time
    if ms_step_eager <= ms_step_graph:
        ms_step, launch = ms_step_eager, "eager (every op of the step in order, steps back to back)"
    else:
        ms_step, launch = ms_step_graph, "hip graph per step (one per input set)"
    kernels = [op_record(op, d, workload) for op, d in zip(wl.ops, per_op)]
    roof_s = sum(op.roofline_seconds() for op in wl.ops)
    probes = []
    if wl.probes:
        per_probe, _ = time_ops(wl.probes, steps, warmup)
        probes = [op_record(op, d, workload) for op, d in zip(wl.probes, per_probe)]
    dom = max(kernels, key=lambda k: k["avg_ms"])
    value = 100.0 * roof_s / (ms_step * 1e-3)
    line = {"metric": METRIC, "value": round(value, 2), "unit": "% of roofline (step)", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
            "ms_per_step_eager": round(ms_step_eager, 5), "ms_per_step_graph": round(ms_step_graph, 5),
            "launch": launch,
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
            "data": "synthetic (seeded generators; no dataset or trained weights)", "config": wl.cfg,
            "roofline": {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                         "unit": dom["unit"], "frac": dom["frac"], "traffic": dom["traffic"],
                         "kernel": dom["kernel"]},
            "step_roofline_ms": round(roof_s * 1e3, 5),
            "kernels": kernels}
    if probes:
        line["kernels_amax_supplied"] = probes
    line["cpu_baseline"] = cpu_baseline(wl, roof_s) if with_cpu and wl.cpu else None
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return line


SUB_KEYS = ("config", "value", "ms_per_step", "ms_per_step_eager", "ms_per_step_graph", "launch", "step_roofline_ms", "roofline", "kernels",
            "kernels_amax_supplied", "cpu_baseline")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="default", choices=["default", *WORKLOADS, "all"],
                    help="default: the headline step with the other configurations in the same line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (HBM counter calibration)")
    ap.add_argument("--ingest-pmc", default=None, metavar="DIR",
                    help="write profiles/hbm_traffic.json from FETCH_SIZE / WRITE_SIZE runs under DIR (no GPU)")
    ap.add_argument("--copy-bytes", type=int, default=512 << 20)
    ap.add_argument("--pmc-command", action="append", default=[], help="command line recorded with the counters")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc, args.copy_bytes, args.pmc_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "sharding the path over several GPUs is designed but not built", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    with_cpu = not args.no_cpu_baseline
    if args.workload == "default":
        import block_scaled_fp4_amax_amd as F
        from block_scaled_fp4_amax_amd import inputs
        line = run("rht", args.steps, args.warmup, with_cpu)
        print(f"# headline step done: {line['ms_per_step']} ms", file=sys.stderr, flush=True)
        line["workloads"] = {}
        for nm in EXTRA_WORKLOADS:
            sub = run(nm, args.steps, args.warmup, with_cpu and nm in CPU_WORKLOADS)
            line["workloads"][sub["config"]["workload"]] = {k: sub[k] for k in SUB_KEYS if k in sub}
            print(f"# {nm} step done: {sub['ms_per_step']} ms", file=sys.stderr, flush=True)
        line["worked_example"] = worked_example_record(F, inputs)
        print(json.dumps(line), flush=True)
        return
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    for nm in names:
        print(json.dumps(run(nm, args.steps, args.warmup, with_cpu)), flush=True)


if __name__ == "__main__":
    main()
