"""block_scaled_fp4_amax_amd -- block-scaled FP4 (E2M1) quantization and the
W4A4 block-scaled GEMM on AMD MI355X (gfx950).

The compute lives in ``libfp4.so`` (hand-written HIP kernels behind the C ABI
of ``include/fp4.h``). This module only marshals arguments:

* ``fp4_quantize``, ``fp4_quantize_noalloc``, ``fp4_dequantize``,
  ``fp4_gemm``, ``fp4_gemm_grouped``, ``fp4_gemm_quantize_output``,
  ``fp4_quantize_workspace``, ``fp4_status_str`` -- the C entry points with
  the same names and argument order (integers for device pointers);
* ``quantize``, ``dequantize``, ``gemm``, ``gemm_grouped``,
  ``gemm_quantize_output`` -- conveniences over torch device
  tensors that allocate outputs with torch, pass the current HIP stream and
  raise ``Fp4Error`` on a non-OK status.

There is no fallback: if ``libfp4.so`` is missing or a call fails, an error is
raised.
"""
from __future__ import annotations

import ctypes
from ctypes import c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p, c_char_p
from dataclasses import dataclass
from pathlib import Path
from typing import Optional

LIB_PATH = Path(__file__).resolve().with_name("libfp4.so")

# fp4_status
FP4_OK = 0
FP4_ERR_INVALID = -1
FP4_ERR_UNSUPPORTED = -2
FP4_ERR_ALIGN = -3
FP4_ERR_DEVICE = -4
FP4_ERR_WORKSPACE = -5
FP4_ERR_HIP = -6
FP4_ERR_SCRATCH = -7
FP4_NOALLOC_SCRATCH_BYTES = 262144
# fp4_format / fp4_dtype
FP4_MXFP4 = 0
FP4_NVFP4 = 1
FP4_F32 = 0
FP4_BF16 = 1
# flags
FP4_FOUR_OVER_SIX = 1
FP4_BLOCK2D = 2
FP4_TRANSPOSE = 4
FP4_STOCHASTIC = 8
FP4_HADAMARD = 16
FP4_SCALE_SEARCH = 32
FP4_TENSOR_SCALE = 64

EXPORTED_SYMBOLS = ("fp4_quantize_workspace", "fp4_quantize", "fp4_quantize_noalloc", "fp4_dequantize", "fp4_gemm",
                    "fp4_gemm_grouped", "fp4_gemm_quantize_output", "fp4_status_str")


class fp4_quant_opts(ctypes.Structure):
    _fields_ = [
        ("size", c_uint32),
        ("format", c_int32),
        ("flags", c_uint32),
        ("rht_signs", c_uint32),
        ("seed", c_uint64),
        ("offset", c_uint64),
        ("amax_in", c_void_p),
    ]


class Fp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fp4_status_str(status)} ({status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libfp4.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m block_scaled_fp4_amax_amd.build` "
                "(or __graft_entry__.build())")
        L = ctypes.CDLL(str(LIB_PATH))
        L.fp4_quantize_workspace.restype = c_size_t
        L.fp4_quantize_workspace.argtypes = [c_int64, c_int64, c_int64, ctypes.POINTER(fp4_quant_opts)]
        L.fp4_quantize.restype = c_int32
        L.fp4_quantize.argtypes = [
            c_void_p, c_int32, c_int64, c_int64, c_int64, c_int64, c_int64, ctypes.POINTER(fp4_quant_opts),
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]
        L.fp4_quantize_noalloc.restype = c_int32
        L.fp4_quantize_noalloc.argtypes = [
            c_void_p, c_int32, c_int64, c_int64, c_int64, c_int64, c_int64, ctypes.POINTER(fp4_quant_opts),
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_void_p]
        L.fp4_dequantize.restype = c_int32
        L.fp4_dequantize.argtypes = [
            c_int32, c_int64, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64,
            c_void_p, c_void_p, c_int32, c_int64, c_int64, c_void_p]
        L.fp4_gemm.restype = c_int32
        L.fp4_gemm.argtypes = [
            c_int32, c_int64, c_int64, c_int64, c_int64,
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            c_void_p, c_int32, c_int64, c_int64, c_void_p]
        L.fp4_gemm_grouped.restype = c_int32
        L.fp4_gemm_grouped.argtypes = [
            c_int32, c_int64, c_void_p, c_int64, c_int64, c_int64,
            c_void_p, c_int64, c_void_p, c_int64, c_void_p,
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            c_void_p, c_int32, c_int64, c_void_p]
        L.fp4_gemm_quantize_output.restype = c_int32
        L.fp4_gemm_quantize_output.argtypes = [
            c_int32, c_int64, c_int64, c_int64, c_int64,
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            ctypes.POINTER(fp4_quant_opts), c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_void_p,
            c_void_p]
        L.fp4_status_str.restype = c_char_p
        L.fp4_status_str.argtypes = [c_int32]
        _lib = L
    return _lib


def make_opts(fmt: int, flags: int = 0, rht_signs: int = 0, seed: int = 0, offset: int = 0,
              amax_in: int = 0) -> fp4_quant_opts:
    o = fp4_quant_opts()
    o.size = ctypes.sizeof(fp4_quant_opts)
    o.format = fmt
    o.flags = flags
    o.rht_signs = rht_signs
    o.seed = seed
    o.offset = offset
    o.amax_in = amax_in or None
    return o


# ---------------------------------------------------------------------------
# raw C entry points (same names, same argument order)
# ---------------------------------------------------------------------------
def fp4_status_str(status: int) -> str:
    return lib().fp4_status_str(status).decode()


def fp4_quantize_workspace(batch, rows, cols, opts: fp4_quant_opts) -> int:
    return lib().fp4_quantize_workspace(batch, rows, cols, ctypes.byref(opts))


def fp4_quantize(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, opts: fp4_quant_opts, codes, ld_codes,
                 batch_stride_codes, scales, ld_scales, batch_stride_scales, tensor_scale, workspace,
                 workspace_bytes, stream) -> int:
    return lib().fp4_quantize(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, ctypes.byref(opts), codes,
                              ld_codes, batch_stride_codes, scales, ld_scales, batch_stride_scales, tensor_scale,
                              workspace, workspace_bytes, stream)


def fp4_quantize_noalloc(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, opts: fp4_quant_opts, codes, ld_codes,
                         batch_stride_codes, scales, ld_scales, batch_stride_scales, tensor_scale, stream) -> int:
    return lib().fp4_quantize_noalloc(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, ctypes.byref(opts), codes,
                                      ld_codes, batch_stride_codes, scales, ld_scales, batch_stride_scales,
                                      tensor_scale, stream)


def fp4_dequantize(fmt, batch, rows, cols, codes, ld_codes, batch_stride_codes, scales, ld_scales,
                   batch_stride_scales, tensor_scale, y, y_dtype, ld_y, batch_stride_y, stream) -> int:
    return lib().fp4_dequantize(fmt, batch, rows, cols, codes, ld_codes, batch_stride_codes, scales, ld_scales,
                                batch_stride_scales, tensor_scale, y, y_dtype, ld_y, batch_stride_y, stream)


def fp4_gemm(fmt, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales, a_scales_group_stride,
             a_tensor_scale, b_codes, ldb, b_group_stride, b_scales, ldb_scales, b_scales_group_stride,
             b_tensor_scale, c, c_dtype, ldc, c_group_stride, stream) -> int:
    return lib().fp4_gemm(fmt, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales,
                          a_scales_group_stride, a_tensor_scale, b_codes, ldb, b_group_stride, b_scales, ldb_scales,
                          b_scales_group_stride, b_tensor_scale, c, c_dtype, ldc, c_group_stride, stream)


def fp4_gemm_quantize_output(fmt, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales,
                             a_scales_group_stride, a_tensor_scale, b_codes, ldb, b_group_stride, b_scales, ldb_scales,
                             b_scales_group_stride, b_tensor_scale, out_opts: fp4_quant_opts, out_codes, ld_out_codes,
                             out_codes_group_stride, out_scales, ld_out_scales, out_scales_group_stride,
                             out_tensor_scale, stream) -> int:
    return lib().fp4_gemm_quantize_output(fmt, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales,
                                          a_scales_group_stride, a_tensor_scale, b_codes, ldb, b_group_stride,
                                          b_scales, ldb_scales, b_scales_group_stride, b_tensor_scale,
                                          ctypes.byref(out_opts), out_codes, ld_out_codes, out_codes_group_stride,
                                          out_scales, ld_out_scales, out_scales_group_stride, out_tensor_scale,
                                          stream)


def fp4_gemm_grouped(fmt, groups, group_offsets, M, N, K, a_codes, lda, a_scales, lda_scales, a_tensor_scale,
                     b_codes, ldb, b_group_stride, b_scales, ldb_scales, b_scales_group_stride, b_tensor_scale, c,
                     c_dtype, ldc, stream) -> int:
    return lib().fp4_gemm_grouped(fmt, groups, group_offsets, M, N, K, a_codes, lda, a_scales, lda_scales,
                                  a_tensor_scale, b_codes, ldb, b_group_stride, b_scales, ldb_scales,
                                  b_scales_group_stride, b_tensor_scale, c, c_dtype, ldc, stream)


# ---------------------------------------------------------------------------
# torch conveniences (allocation + current stream only)
# ---------------------------------------------------------------------------
def scale_pitch(n_blocks: int) -> int:
    """Scale-row pitch in bytes that fp4_gemm accepts: rounded up to 16."""
    return (n_blocks + 15) // 16 * 16


def code_pitch(n_bytes: int) -> int:
    """Code-row pitch in bytes: rounded up to 128 (one cache line), so that
    every row starts on a line and no store of a row shares a line with the
    next row (rows of 1440 bytes otherwise straddle lines)."""
    return (n_bytes + 127) // 128 * 128


@dataclass
class Quantized:
    """Packed FP4 tensor as written by fp4_quantize. Shapes carry an optional
    leading batch dimension: codes [.., R, C/2], scales [.., R, C/blk],
    tensor_scale [batch] (NVFP4) or None. `codes` and `scales` may be views
    whose row pitch (stride(-2)) exceeds C/2 or C/blk: quantize() pads code
    rows to code_pitch() and scale rows to scale_pitch()."""
    fmt: int
    codes: "torch.Tensor"
    scales: "torch.Tensor"
    tensor_scale: Optional["torch.Tensor"]

    @property
    def block(self) -> int:
        return 16 if self.fmt == FP4_NVFP4 else 32

    @property
    def shape(self):
        return (*self.codes.shape[:-1], self.codes.shape[-1] * 2)


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return {"mxfp4": FP4_MXFP4, "nvfp4": FP4_NVFP4}[fmt.lower()]
    return int(fmt)


def _stream(stream):
    import torch
    return stream if stream is not None else torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != FP4_OK:
        raise Fp4Error(status, where)


def quantize(x, fmt="nvfp4", *, four_over_six=False, block2d=False, transpose=False, stochastic=False,
             hadamard=False, scale_search=False, tensor_scale=False, rht_signs=0, seed=0, offset=0, amax=None,
             stream=None) -> Quantized:
    """Quantize a [rows, cols] or [batch, rows, cols] bf16/fp32 device tensor
    (tensor_scale: the NVFP4 whole-tensor mode, FP4_TENSOR_SCALE)."""
    import torch
    fmt = _fmt(fmt)
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    if x3.dim() != 3:
        raise ValueError("quantize expects a 2-D or 3-D tensor")
    x3 = x3.contiguous()
    batch, rows, cols = x3.shape
    dt = {torch.bfloat16: FP4_BF16, torch.float32: FP4_F32}[x3.dtype]
    flags = ((FP4_FOUR_OVER_SIX if four_over_six else 0) | (FP4_BLOCK2D if block2d else 0)
             | (FP4_TRANSPOSE if transpose else 0) | (FP4_STOCHASTIC if stochastic else 0)
             | (FP4_HADAMARD if hadamard else 0) | (FP4_SCALE_SEARCH if scale_search else 0)
             | (FP4_TENSOR_SCALE if tensor_scale else 0))
    amax_t = None
    if amax is not None:
        amax_t = torch.as_tensor(amax, dtype=torch.float32, device=x3.device).reshape(-1).contiguous()
    opts = make_opts(fmt, flags, rht_signs, seed, offset, amax_t.data_ptr() if amax_t is not None else 0)
    R, C = (cols, rows) if transpose else (rows, cols)
    blk = 16 if fmt == FP4_NVFP4 else 32
    dev = x3.device
    ldc = code_pitch(C // 2)
    codes = torch.empty((batch, R, ldc), dtype=torch.uint8, device=dev)[:, :, : C // 2]
    lds = scale_pitch(C // blk)
    scales_buf = torch.empty((batch, R, lds), dtype=torch.uint8, device=dev)
    scales = scales_buf[:, :, : C // blk]
    ts = torch.empty((batch,), dtype=torch.float32, device=dev) if fmt == FP4_NVFP4 else None
    ws_bytes = fp4_quantize_workspace(batch, rows, cols, opts)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev) if ws_bytes else None
    st = fp4_quantize(x3.data_ptr(), dt, batch, rows, cols, cols, rows * cols, opts, codes.data_ptr(), ldc,
                      R * ldc, scales_buf.data_ptr(), lds, R * lds,
                      ts.data_ptr() if ts is not None else None, ws.data_ptr() if ws is not None else None,
                      ws_bytes, _stream(stream))
    _check(st, "fp4_quantize")
    if squeeze:
        codes, scales = codes[0], scales[0]
    return Quantized(fmt, codes, scales, ts)


def _check_scales(scales):
    """Scales are passed by base pointer and row / batch pitch: the last dim
    must be dense."""
    if scales.stride(-1) != 1:
        raise ValueError("scale rows must be contiguous")


def _check_codes(codes):
    """Codes likewise: dense rows, any row / batch pitch."""
    if codes.stride(-1) != 1:
        raise ValueError("code rows must be contiguous")


def dequantize(q: Quantized, dtype=None, stream=None):
    import torch
    dtype = dtype or torch.float32
    codes = q.codes if q.codes.dim() == 3 else q.codes.unsqueeze(0)
    scales = q.scales if q.scales.dim() == 3 else q.scales.unsqueeze(0)
    batch, rows, half = codes.shape
    cols = half * 2
    y = torch.empty((batch, rows, cols), dtype=dtype, device=codes.device)
    dt = {torch.bfloat16: FP4_BF16, torch.float32: FP4_F32}[dtype]
    _check_scales(scales)
    _check_codes(codes)
    st = fp4_dequantize(q.fmt, batch, rows, cols, codes.data_ptr(), codes.stride(1), codes.stride(0),
                        scales.data_ptr(),
                        scales.stride(1), scales.stride(0),
                        q.tensor_scale.data_ptr() if q.tensor_scale is not None else None, y.data_ptr(), dt, cols,
                        rows * cols, _stream(stream))
    _check(st, "fp4_dequantize")
    return y if q.codes.dim() == 3 else y[0]


def gemm(a: Quantized, b: Quantized, out_dtype=None, stream=None):
    """C[g] = deq(A[g]) @ deq(B[g])^T with A [.., M, K] and B [.., N, K]."""
    import torch
    out_dtype = out_dtype or torch.float32
    if a.fmt != b.fmt:
        raise ValueError("operands must share a format")
    ac = a.codes if a.codes.dim() == 3 else a.codes.unsqueeze(0)
    asc = a.scales if a.scales.dim() == 3 else a.scales.unsqueeze(0)
    bc = b.codes if b.codes.dim() == 3 else b.codes.unsqueeze(0)
    bsc = b.scales if b.scales.dim() == 3 else b.scales.unsqueeze(0)
    G, M, half = ac.shape
    Gb, N, halfb = bc.shape
    if G != Gb or half != halfb:
        raise ValueError("operand shapes do not match")
    K = half * 2
    c = torch.empty((G, M, N), dtype=out_dtype, device=ac.device)
    ct = {torch.bfloat16: FP4_BF16, torch.float32: FP4_F32}[out_dtype]
    _check_scales(asc)
    _check_scales(bsc)
    _check_codes(ac)
    _check_codes(bc)
    st = fp4_gemm(a.fmt, G, M, N, K, ac.data_ptr(), ac.stride(1), ac.stride(0), asc.data_ptr(), asc.stride(1),
                  asc.stride(0), a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                  bc.data_ptr(), bc.stride(1), bc.stride(0), bsc.data_ptr(), bsc.stride(1), bsc.stride(0),
                  b.tensor_scale.data_ptr() if b.tensor_scale is not None else None, c.data_ptr(), ct, N, M * N,
                  _stream(stream))
    _check(st, "fp4_gemm")
    return c if a.codes.dim() == 3 else c[0]


def gemm_quantize_output(a: Quantized, b: Quantized, fmt="nvfp4", *, four_over_six=False, stochastic=False,
                         hadamard=False, scale_search=False, rht_signs=0, seed=0, offset=0, amax=None,
                         stream=None) -> Quantized:
    """deq(A[g]) @ deq(B[g])^T quantized along its rows in the GEMM's epilogue
    (format `fmt`, options as for quantize); NVFP4 needs `amax`, the tensor
    amax per group that S_t derives from."""
    import torch
    if a.fmt != b.fmt:
        raise ValueError("operands must share a format")
    ac = a.codes if a.codes.dim() == 3 else a.codes.unsqueeze(0)
    asc = a.scales if a.scales.dim() == 3 else a.scales.unsqueeze(0)
    bc = b.codes if b.codes.dim() == 3 else b.codes.unsqueeze(0)
    bsc = b.scales if b.scales.dim() == 3 else b.scales.unsqueeze(0)
    G, M, half = ac.shape
    Gb, N, halfb = bc.shape
    if G != Gb or half != halfb:
        raise ValueError("operand shapes do not match")
    qfmt = _fmt(fmt)
    flags = ((FP4_FOUR_OVER_SIX if four_over_six else 0) | (FP4_STOCHASTIC if stochastic else 0)
             | (FP4_HADAMARD if hadamard else 0) | (FP4_SCALE_SEARCH if scale_search else 0))
    amax_t = None
    if amax is not None:
        amax_t = torch.as_tensor(amax, dtype=torch.float32, device=ac.device).reshape(-1).contiguous()
    opts = make_opts(qfmt, flags, rht_signs, seed, offset, amax_t.data_ptr() if amax_t is not None else 0)
    blk = 16 if qfmt == FP4_NVFP4 else 32
    dev = ac.device
    ldq = code_pitch(N // 2)
    codes = torch.empty((G, M, ldq), dtype=torch.uint8, device=dev)[:, :, : N // 2]
    lds = scale_pitch(N // blk)
    scales_buf = torch.empty((G, M, lds), dtype=torch.uint8, device=dev)
    ts = torch.empty((G,), dtype=torch.float32, device=dev) if qfmt == FP4_NVFP4 else None
    _check_scales(asc)
    _check_scales(bsc)
    _check_codes(ac)
    _check_codes(bc)
    st = fp4_gemm_quantize_output(a.fmt, G, M, N, half * 2, ac.data_ptr(), ac.stride(1), ac.stride(0),
                                  asc.data_ptr(), asc.stride(1), asc.stride(0),
                                  a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                                  bc.data_ptr(), bc.stride(1), bc.stride(0), bsc.data_ptr(), bsc.stride(1),
                                  bsc.stride(0), b.tensor_scale.data_ptr() if b.tensor_scale is not None else None,
                                  opts, codes.data_ptr(), ldq, M * ldq, scales_buf.data_ptr(), lds, M * lds,
                                  ts.data_ptr() if ts is not None else None, _stream(stream))
    _check(st, "fp4_gemm_quantize_output")
    scales = scales_buf[:, :, : N // blk]
    if a.codes.dim() == 2:
        codes, scales = codes[0], scales[0]
    return Quantized(qfmt, codes, scales, ts)


def gemm_grouped(a: Quantized, b: Quantized, offsets, out_dtype=None, stream=None):
    """Mixture-of-experts grouped GEMM: rows offsets[g]:offsets[g + 1] of
    A [M, K] times B[g] [N, K]^T, into C [M, N]. `offsets` is a device int32
    tensor of groups + 1 entries (e.g. a router's cumulative counts)."""
    import torch
    out_dtype = out_dtype or torch.float32
    if a.fmt != b.fmt:
        raise ValueError("operands must share a format")
    if a.codes.dim() != 2:
        raise ValueError("A must be one [M, K] matrix")
    bc = b.codes if b.codes.dim() == 3 else b.codes.unsqueeze(0)
    bsc = b.scales if b.scales.dim() == 3 else b.scales.unsqueeze(0)
    G, N, half = bc.shape
    M, halfa = a.codes.shape
    if half != halfa:
        raise ValueError("operand shapes do not match")
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or offsets.numel() != G + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int32 vector of groups + 1 entries")
    offsets = offsets.contiguous()
    c = torch.empty((M, N), dtype=out_dtype, device=a.codes.device)
    ct = {torch.bfloat16: FP4_BF16, torch.float32: FP4_F32}[out_dtype]
    _check_scales(a.scales.unsqueeze(0))
    _check_scales(bsc)
    _check_codes(a.codes)
    _check_codes(bc)
    st = fp4_gemm_grouped(a.fmt, G, offsets.data_ptr(), M, N, half * 2, a.codes.data_ptr(), a.codes.stride(0),
                          a.scales.data_ptr(), a.scales.stride(0),
                          a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                          bc.data_ptr(), bc.stride(1), bc.stride(0), bsc.data_ptr(), bsc.stride(1), bsc.stride(0),
                          b.tensor_scale.data_ptr() if b.tensor_scale is not None else None, c.data_ptr(), ct, N,
                          _stream(stream))
    _check(st, "fp4_gemm_grouped")
    return c
