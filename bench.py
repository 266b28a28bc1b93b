#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 hot path on one MI355X.

A step is one pass of the workload's whole path over one batch of seeded
synthetic input already resident in HBM. The default workload is the W4A4
linear layer: NVFP4 four-over-six quantization of the activations
[2048, 4096] and of the weight [4096, 4096] (each with its tensor-amax
pre-pass), then the NVFP4 GEMM to a [2048, 4096] bf16 output.

Timing: W untimed warm-up steps, then K steps between two device
synchronisations, with HIP events (torch.cuda.Event on the stream the kernels
run on) around the whole region and around every op inside it. Inputs rotate
over enough copies (>= 600 MB) that the 256 MB Infinity Cache cannot serve
them from one step to the next.

Output: one JSON line. `value` is the step's roofline time (sum over its ops
of algorithmic bytes / 8 TB/s for codec scans, flops / dense matrix peak for
the GEMM) as a percentage of the measured step time. `roofline` describes the
op that takes most of the step; `kernels` lists every op. `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload (single
thread), scaled to the full step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
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
def wl_w4a4_linear(F, inputs):
    d = inputs.w4a4_linear(device="cuda")
    n = n_sets(d["a"].numel() * 2 + d["w"].numel() * 2)
    qa = QuantCall(F, copies(d["a"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
    gm = GemmCall(F, qa, qw, torch.bfloat16)
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", "gemm_fp4_kernel<true, 128, 4, 1, false>", "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s")]
    cfg = {"workload": "w4a4_linear_nvfp4_four_over_six", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "bf16", "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", lambda: cpu_w4a4(d)


def wl_moe(F, inputs):
    d = inputs.moe_mxfp4(device="cuda")
    n = n_sets(d["w"].numel() * 2 + d["x"].numel() * 2)
    qw = QuantCall(F, copies(d["w"], n), F.FP4_MXFP4, F.FP4_TRANSPOSE)
    qx = QuantCall(F, copies(d["x"], n), F.FP4_MXFP4, 0)
    gm = GemmCall(F, qx, qw, torch.bfloat16)
    ops = [Op("quantize W^T mxfp4 32x[2880x5760]", "quant_cols_kernel", "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("quantize X mxfp4 32x[512x2880]", "quant_rows_kernel", "hbm", qx.bytes(),
              PEAK_HBM_GBS, qx, "GB/s"),
           Op("grouped gemm mxfp4 (scaled FP4 MFMA)", "gemm_fp4_kernel<false, 256, 4, 1, false>", "mfma",
              gm.flops(), PEAK_TFLOPS["fp4"], gm, "TFLOP/s")]
    cfg = {"workload": "moe_mxfp4_grouped", "experts": 32, "M": 512, "N": 5760, "K": 2880, "output": "bf16",
           "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (mxfp4); fp4 MFMA, f32 accumulate", None


def wl_training(F, inputs):
    d = inputs.training(device="cuda")
    n = n_sets(d["w"].numel() * 4)
    # W and W^T read their own copies: a second read of the same tensor right
    # after the first would be served from the 256 MB Infinity Cache
    ws, ws2, gs = copies(d["w"], n), copies(d["w"], n), copies(d["grad"], n)
    f = F.FP4_FOUR_OVER_SIX | F.FP4_BLOCK2D
    q1 = QuantCall(F, ws, F.FP4_NVFP4, f)
    q2 = QuantCall(F, ws2, F.FP4_NVFP4, f | F.FP4_TRANSPOSE)
    q3 = QuantCall(F, gs, F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX | F.FP4_STOCHASTIC, seed=d["sr_seed"])
    ops = [Op("quantize W nvfp4 2D 4/6", "quant_rows_kernel", "hbm", q1.bytes(), PEAK_HBM_GBS, q1, "GB/s", lane=1),
           Op("quantize W^T nvfp4 2D 4/6", "quant_cols_kernel", "hbm", q2.bytes(), PEAK_HBM_GBS, q2, "GB/s", lane=2),
           Op("quantize G nvfp4 4/6 stochastic", "quant_rows_kernel", "hbm", q3.bytes(),
              PEAK_HBM_GBS, q3, "GB/s", lane=3)]
    cfg = {"workload": "training_quantize_8192", "shape": [8192, 8192], "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4), f32 scale arithmetic", None


def wl_rht(F, inputs):
    d = inputs.rht_activation(device="cuda")
    n = n_sets(d["x"].numel() * 2 + d["w"].numel() * 2)
    f = F.FP4_FOUR_OVER_SIX | F.FP4_HADAMARD
    qx = QuantCall(F, copies(d["x"], n), F.FP4_NVFP4, f, signs=d["signs"])
    qw = QuantCall(F, copies(d["w"], n), F.FP4_NVFP4, f | F.FP4_TRANSPOSE, signs=d["signs"])
    gm = GemmCall(F, qx, qw, torch.bfloat16)
    ops = [Op("quantize X nvfp4 4/6 RHT", "quant_rows_kernel", "hbm", qx.bytes(), PEAK_HBM_GBS, qx, "GB/s", lane=1),
           Op("quantize W^T nvfp4 4/6 RHT", "quant_cols_kernel", "hbm", qw.bytes(), PEAK_HBM_GBS, qw, "GB/s", lane=2),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", "gemm_fp4_kernel<true, 128, 4, 1, false>", "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s")]
    cfg = {"workload": "rht_activation_nvfp4", "M": 16384, "N": 12288, "K": 4096, "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", None


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
    ops = [Op("quantize dY nvfp4 4/6 stochastic", "quant_rows_kernel", "hbm", qg.bytes(),
              PEAK_HBM_GBS, qg, "GB/s", lane=1),
           Op("quantize W^T nvfp4 2D 4/6", "quant_cols_kernel", "hbm", qwt.bytes(), PEAK_HBM_GBS, qwt, "GB/s", lane=2),
           Op("dgrad gemm nvfp4 dX = dY W", "gemm_fp4_kernel<true, 128, 4, 1, false>", "mfma", gd.flops(),
              PEAK_TFLOPS["f16"], gd, "TFLOP/s"),
           Op("quantize dY^T nvfp4 4/6 stochastic", "quant_cols_kernel", "hbm", qgt.bytes(), PEAK_HBM_GBS, qgt,
              "GB/s", lane=1),
           Op("quantize X^T nvfp4 4/6", "quant_cols_kernel", "hbm", qxt.bytes(), PEAK_HBM_GBS, qxt, "GB/s", lane=2),
           Op("wgrad gemm nvfp4 dW = dY^T X", "gemm_fp4_kernel<true, 128, 4, 1, false>", "mfma", gw.flops(),
              PEAK_TFLOPS["f16"], gw, "TFLOP/s")]
    cfg = {"workload": "training_backward_nvfp4_8192", "M": 8192, "N": 8192, "K": 8192,
           "gradient": "8192x8192 bf16 Laplace(0,1e-3)", "weight": "8192x8192 bf16 N(0,0.02)",
           "activations": "8192x8192 bf16 N(0,1)", "output": "bf16", "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", None


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
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4, output quantized to nvfp4 4/6 in the epilogue", "gemm_fp4_kernel<true, 128, 4, 3, false>",
              "mfma", gq.flops(), PEAK_TFLOPS["f16"], gq, "TFLOP/s")]
    cfg = {"workload": "w4a4_linear_nvfp4_fused_output_quantize", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "nvfp4 4/6 codes + scales, amax supplied", "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", None


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
    ops = [Op("quantize A nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qa.bytes(),
              PEAK_HBM_GBS, qa, "GB/s"),
           Op("quantize W nvfp4 4/6 (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("gemm nvfp4 (exact fp16 dequant + fp16 MFMA)", "gemm_fp4_kernel<true, 128, 4, 1, false>", "mfma",
              gm.flops(), PEAK_TFLOPS["f16"], gm, "TFLOP/s"),
           Op("quantize C nvfp4 4/6 (amax supplied)", "quant_rows_kernel", "hbm", qc.bytes(), PEAK_HBM_GBS, qc,
              "GB/s")]
    cfg = {"workload": "w4a4_linear_nvfp4_unfused_output_quantize", "M": 2048, "N": 4096, "K": 4096,
           "activations": "2048x4096 bf16 N(0,1), 1% columns x30", "weight": "4096x4096 bf16 N(0,0.02)",
           "output": "bf16 C, then nvfp4 4/6 codes + scales, amax supplied", "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (nvfp4); f16 MFMA, f32 accumulate", None


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
    ops = [Op("quantize W nvfp4 scale search (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm",
              qs.bytes(), PEAK_HBM_GBS, qs, "GB/s", lane=1),
           Op("quantize W nvfp4 2D scale search (amax pre-pass + quantize)", "amax_kernel+quant_rows_kernel", "hbm",
              q2.bytes(), PEAK_HBM_GBS, q2, "GB/s", lane=2),
           Op("quantize W mxfp4 4/6 exponent pair", "quant_rows_kernel", "hbm", qm.bytes(),
              PEAK_HBM_GBS, qm, "GB/s", lane=3)]
    cfg = {"workload": "scale_search_8192", "shape": [8192, 8192], "weight": "8192x8192 bf16 N(0,0.02)",
           "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes, f32 scale arithmetic", None


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
    ops = [Op("quantize W^T mxfp4 32x[2880x5760]", "quant_cols_kernel", "hbm", qw.bytes(),
              PEAK_HBM_GBS, qw, "GB/s"),
           Op("quantize routed X mxfp4 [16384x2880]", "quant_rows_kernel", "hbm", qx.bytes(), PEAK_HBM_GBS, qx,
              "GB/s"),
           Op("grouped gemm mxfp4, router row counts", "gemm_fp4_kernel<false, 256, 4, 1, true>", "mfma",
              gm.flops(), PEAK_TFLOPS["fp4"], gm, "TFLOP/s")]
    cfg = {"workload": "moe_mxfp4_routed", "experts": 32, "tokens": 4096, "top_k": 4, "rows": int(d["offsets"][-1]),
           "rows_per_expert": [int(v) for v in d["counts"]], "N": 5760, "K": 2880, "output": "bf16",
           "input_sets_rotated": n}
    return ops, cfg, "fp4 e2m1 codes (mxfp4); fp4 MFMA, f32 accumulate", None


WORKLOADS = {"w4a4_linear": wl_w4a4_linear, "moe": wl_moe, "training": wl_training, "rht": wl_rht,
             "training_backward": wl_training_backward, "moe_routed": wl_moe_routed, "w4a4_fused": wl_w4a4_fused,
             "w4a4_unfused_chain": wl_w4a4_unfused_chain, "scale_search": wl_scale_search}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, single thread, bounded sample
# ---------------------------------------------------------------------------
def cpu_w4a4(d):
    from threadpoolctl import threadpool_limits

    from block_scaled_fp4_amax_amd import inputs
    from oracle import oracle as O
    a = inputs.bf16_bits(d["a"].cpu())
    w = inputs.bf16_bits(d["w"].cpu())
    M, K = a.shape
    N = w.shape[0]
    rows = 1024
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        qa = O.quantize(a, O.NVFP4, flags=O.FOUR_OVER_SIX)
        t1 = time.perf_counter()
        qw = O.quantize(w, O.NVFP4, flags=O.FOUR_OVER_SIX)
        t2 = time.perf_counter()
        da = O.dequantize(O.NVFP4, qa["codes"][:rows], qa["scales"][:rows], qa["tensor_scale"])
        dw = O.dequantize(O.NVFP4, qw["codes"], qw["scales"], qw["tensor_scale"])
        O.gemm_reference(da, dw)
        t3 = time.perf_counter()
    t_step = (t1 - t0) + (t2 - t1) + (t3 - t2) * (M / rows)
    return {"seconds_measured": t3 - t0, "step_seconds_extrapolated": t_step,
            "sample": f"oracle NVFP4 4/6 quantize of all of A [{M},{K}] and W [{N},{K}] "
                      f"(incl. tensor amax), dequantize + float64 matmul of {rows} of {M} output rows, "
                      f"scaled by {M // rows} to the full GEMM",
            "quantize_GBps": (quant_bytes(M * K, 2, 16, True) + quant_bytes(N * K, 2, 16, True)) / (t2 - t0) / 1e9,
            "gemm_GFLOPs": 2.0 * rows * N * K / (t3 - t2) / 1e9}


# ---------------------------------------------------------------------------
KERNEL_SOURCES = {  # device sources each kernel family is built from
    "gemm": ["gemm.hip", "fp4_device.h", "launch.h"],
    "quant": ["quantize.hip", "quant_common.h", "fp4_device.h", "launch.h"],
    "dequant": ["dequantize.hip", "fp4_device.h", "launch.h"],
}


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


def traffic_for(op_kernel, workload):
    """HBM bytes per launch of one kernel, from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources; else
    None (also for ops made of several kernels)."""
    p = ROOT / "profiles" / "hbm_traffic.json"
    if not p.exists() or "+" in op_kernel:
        return None
    try:
        t = json.loads(p.read_text())
    except ValueError:
        return None
    e = t.get("workloads", {}).get(workload, {}).get(op_kernel)
    if not e or e.get("source_digest") != source_digest(op_kernel):
        return None
    return e.get("bytes_per_launch")


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
            if k not in wr:
                continue
            fb = float(np.mean(fe[k])) * 1024.0 * f_fetch
            wb = float(np.mean(wr[k])) * 1024.0 * f_write
            ent[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                      "dispatches": len(fe[k]), "source_digest": source_digest(k) if "<" in k else None}
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


def run(workload, steps, warmup, with_cpu):
    import block_scaled_fp4_amax_amd as F
    from block_scaled_fp4_amax_amd import inputs
    F.lib()
    torch.manual_seed(0)
    ops, cfg, dtype, cpu_fn = WORKLOADS[workload](F, inputs)
    torch.cuda.synchronize()
    for i in range(warmup):
        for op in ops:
            op.launch(i)
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
           for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        for j, op in enumerate(ops):
            evs[i][j][0].record()
            op.launch(i)
            evs[i][j][1].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_step_eager = t_start.elapsed_time(t_end) / steps
    ms_step = graph_step_ms(ops, steps, warmup)
    kernels = []
    roof_s = 0.0
    for j, op in enumerate(ops):
        d = [evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)]
        avg_ms = float(np.mean(d))
        achieved = op.work / (avg_ms * 1e-3) / (1e9 if op.unit == "GB/s" else 1e12)
        traffic = traffic_for(op.kernel, workload)
        kernels.append({"op": op.name, "kernel": op.kernel, "bound": op.bound, "avg_ms": round(avg_ms, 5),
                        "achieved": round(achieved, 2), "peak": op.peak, "unit": op.unit,
                        "frac": round(achieved / op.peak, 4), "work_per_launch": op.work,
                        "traffic": traffic})
        roof_s += op.roofline_seconds()
    dom = max(kernels, key=lambda k: k["avg_ms"])
    value = 100.0 * roof_s / (ms_step * 1e-3)
    line = {"metric": METRIC, "value": round(value, 2), "unit": "% of roofline (step)", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
            "ms_per_step_eager": round(ms_step_eager, 5), "launch": "hip graph per step (one per input set)",
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded generators; no dataset or trained weights)", "config": cfg,
            "roofline": {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                         "unit": dom["unit"], "frac": dom["frac"], "traffic": dom["traffic"],
                         "kernel": dom["kernel"]},
            "kernels": kernels}
    if with_cpu and cpu_fn is not None:
        c = cpu_fn()
        line["cpu_baseline"] = {"value": round(100.0 * roof_s / c["step_seconds_extrapolated"], 6),
                                "unit": "% of roofline (step)", "cores": 1, "kind": "oracle",
                                "sample": c["sample"], "step_seconds": round(c["step_seconds_extrapolated"], 3),
                                "quantize_GBps": round(c["quantize_GBps"], 4),
                                "gemm_GFLOPs": round(c["gemm_GFLOPs"], 3),
                                "host": f"{os.cpu_count()} logical CPUs visible"}
    else:
        line["cpu_baseline"] = None
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="w4a4_linear", choices=[*WORKLOADS, "all"])
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
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    for nm in names:
        line = run(nm, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
