"""The C-ABI boundary on the host: the library loads, exports every entry
point include/fp4.h declares, and rejects bad arguments with the documented
status before touching HIP. No kernel runs here: device pointers are fake,
and the only calls that get past validation (-> FP4_ERR_DEVICE) run only on
a machine without a GPU."""
import ctypes
import re
from pathlib import Path

import pytest
import torch

ROOT = Path(__file__).resolve().parents[1]
FAKE = 0x7F0000000000  # 256-byte aligned fake device address, never dereferenced
NO_GPU = not torch.cuda.is_available()
cpu_only = pytest.mark.skipif(not NO_GPU, reason="would launch on fake pointers: host-only check")


def header_functions():
    text = (ROOT / "include" / "fp4.h").read_text()
    return re.findall(r"^(?:const char\*|size_t|fp4_status)\s+(fp4_\w+)\s*\(", text, re.M)


def test_library_exports_every_declared_entry_point(fp4):
    names = header_functions()
    assert sorted(names) == sorted(fp4.EXPORTED_SYMBOLS)
    for n in names:
        assert getattr(fp4.lib(), n) is not None


def test_status_strings(fp4):
    for s in range(-7, 1):
        txt = fp4.fp4_status_str(s)
        assert txt.startswith("FP4_")
    assert "unknown" in fp4.fp4_status_str(-99)


def test_opts_struct_layout_matches_header(fp4):
    assert ctypes.sizeof(fp4.fp4_quant_opts) == 40
    assert fp4.fp4_quant_opts.amax_in.offset == 32


def q(fp4, opts, x=FAKE, dt=1, batch=1, rows=64, cols=64, ld_x=None, bsx=0, codes=FAKE, ldc=None, bsc=0,
      scales=FAKE, lds=None, bss=0, ts=FAKE, ws=FAKE, ws_bytes=1 << 20):
    tr = opts.flags & fp4.FP4_TRANSPOSE
    R, C = (cols, rows) if tr else (rows, cols)
    blk = 16 if opts.format == fp4.FP4_NVFP4 else 32
    return fp4.fp4_quantize(x, dt, batch, rows, cols, cols if ld_x is None else ld_x, bsx, opts, codes,
                            C // 2 if ldc is None else ldc, bsc, scales, C // blk if lds is None else lds, bss, ts,
                            ws, ws_bytes, None)


def test_quantize_option_errors(fp4):
    o = fp4.make_opts(fp4.FP4_NVFP4)
    assert fp4.lib().fp4_quantize(FAKE, 1, 1, 64, 64, 64, 0, None, FAKE, 32, 0, FAKE, 4, 0, FAKE, FAKE, 1 << 20,
                                  None) == fp4.FP4_ERR_INVALID
    bad = fp4.make_opts(fp4.FP4_NVFP4)
    bad.size = 8
    assert q(fp4, bad) == fp4.FP4_ERR_INVALID
    assert q(fp4, fp4.make_opts(7)) == fp4.FP4_ERR_INVALID
    assert q(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=fp4.FP4_SCALE_SEARCH)) == fp4.FP4_ERR_UNSUPPORTED
    assert q(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=fp4.FP4_BLOCK2D)) == fp4.FP4_ERR_UNSUPPORTED
    f = fp4.FP4_BLOCK2D | fp4.FP4_HADAMARD | fp4.FP4_TRANSPOSE
    assert q(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=f)) == fp4.FP4_ERR_UNSUPPORTED
    assert q(fp4, o, dt=5) == fp4.FP4_ERR_INVALID
    ts = fp4.FP4_TENSOR_SCALE
    assert q(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=ts)) == fp4.FP4_ERR_UNSUPPORTED
    for other in (fp4.FP4_FOUR_OVER_SIX, fp4.FP4_SCALE_SEARCH, fp4.FP4_BLOCK2D):
        assert q(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=ts | other)) == fp4.FP4_ERR_UNSUPPORTED
    assert q(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=128)) == fp4.FP4_ERR_INVALID


def test_quantize_shape_errors(fp4):
    nv = fp4.make_opts(fp4.FP4_NVFP4)
    mx = fp4.make_opts(fp4.FP4_MXFP4)
    assert q(fp4, nv, cols=24) == fp4.FP4_ERR_INVALID               # cols % 16
    assert q(fp4, mx, cols=48) == fp4.FP4_ERR_INVALID               # cols % 32
    tr = fp4.make_opts(fp4.FP4_NVFP4, flags=fp4.FP4_TRANSPOSE)
    assert q(fp4, tr, rows=24, cols=64) == fp4.FP4_ERR_INVALID      # blocks run down the 24 rows
    assert q(fp4, tr, rows=64, cols=36) == fp4.FP4_ERR_INVALID      # source columns % 8
    b2 = fp4.make_opts(fp4.FP4_NVFP4, flags=fp4.FP4_BLOCK2D)
    assert q(fp4, b2, rows=40, cols=64) == fp4.FP4_ERR_INVALID      # tile rows % 16
    assert q(fp4, nv, rows=-1) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, batch=70000) == fp4.FP4_ERR_UNSUPPORTED


def test_quantize_empty_is_a_noop(fp4):
    nv = fp4.make_opts(fp4.FP4_NVFP4)
    for kw in ({"rows": 0}, {"cols": 0}, {"batch": 0}):
        assert q(fp4, nv, x=0, codes=0, scales=0, ts=0, ws=0, ws_bytes=0, **kw) == fp4.FP4_OK


def test_quantize_pointer_stride_alignment_errors(fp4):
    nv = fp4.make_opts(fp4.FP4_NVFP4)
    assert q(fp4, nv, x=0) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, codes=0) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, scales=0) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, ts=0) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, ld_x=32) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, ldc=16) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, lds=2) == fp4.FP4_ERR_INVALID
    assert q(fp4, nv, batch=2, bsc=100) == fp4.FP4_ERR_INVALID       # overlapping outputs
    assert q(fp4, nv, x=FAKE + 8) == fp4.FP4_ERR_ALIGN
    assert q(fp4, nv, ld_x=68) == fp4.FP4_ERR_ALIGN                  # 136-byte bf16 rows
    assert q(fp4, nv, codes=FAKE + 4) == fp4.FP4_ERR_ALIGN
    assert q(fp4, nv, ldc=36) == fp4.FP4_ERR_ALIGN


def test_workspace_size_and_errors(fp4):
    nv = fp4.make_opts(fp4.FP4_NVFP4)
    need = fp4.fp4_quantize_workspace(1, 64, 64, nv)
    assert need > 0 and need % 4 == 0
    assert fp4.fp4_quantize_workspace(3, 64, 64, nv) == 3 * need
    assert fp4.fp4_quantize_workspace(1, 64, 64, fp4.make_opts(fp4.FP4_MXFP4)) == 0
    assert fp4.fp4_quantize_workspace(1, 64, 64, fp4.make_opts(fp4.FP4_NVFP4, amax_in=FAKE)) == 0
    assert fp4.fp4_quantize_workspace(1, 64, 24, nv) == 0           # rejected shape
    assert q(fp4, nv, ws=0, ws_bytes=0) == fp4.FP4_ERR_WORKSPACE
    assert q(fp4, nv, ws_bytes=need - 4) == fp4.FP4_ERR_WORKSPACE
    assert q(fp4, nv, ws=FAKE + 4) == fp4.FP4_ERR_ALIGN


def qn(fp4, opts, batch=1, rows=64, cols=64, x=FAKE, codes=FAKE, scales=FAKE, ts=FAKE):
    tr = opts.flags & fp4.FP4_TRANSPOSE
    R, C = (cols, rows) if tr else (rows, cols)
    blk = 16 if opts.format == fp4.FP4_NVFP4 else 32
    return fp4.fp4_quantize_noalloc(x, 1, batch, rows, cols, cols, rows * cols, opts, codes, C // 2, R * (C // 2),
                                    scales, C // blk, R * (C // blk), ts, None)


def test_noalloc_validation_and_scratch_limit(fp4):
    nv = fp4.make_opts(fp4.FP4_NVFP4)
    assert fp4.FP4_NOALLOC_SCRATCH_BYTES == 262144
    # the same argument checks as fp4_quantize
    assert qn(fp4, nv, cols=24) == fp4.FP4_ERR_INVALID
    assert qn(fp4, nv, x=0) == fp4.FP4_ERR_INVALID
    assert qn(fp4, nv, x=FAKE + 8) == fp4.FP4_ERR_ALIGN
    assert qn(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=fp4.FP4_BLOCK2D)) == fp4.FP4_ERR_UNSUPPORTED
    for kw in ({"rows": 0}, {"batch": 0}):
        assert qn(fp4, nv, x=0, codes=0, scales=0, ts=0, **kw) == fp4.FP4_OK
    # an NVFP4 item without amax_in needs at most 1025 words: 63 items fit,
    # 64 of the largest size do not, and are refused before any HIP call
    big = (8192, 8192)
    per_item = fp4.fp4_quantize_workspace(1, *big, nv)
    assert per_item == 1025 * 4
    assert 63 * per_item <= fp4.FP4_NOALLOC_SCRATCH_BYTES < 64 * per_item
    assert qn(fp4, nv, batch=64, rows=big[0], cols=big[1]) == fp4.FP4_ERR_SCRATCH


@cpu_only
def test_valid_noalloc_without_gfx950_reports_device(fp4):
    assert qn(fp4, fp4.make_opts(fp4.FP4_NVFP4)) == fp4.FP4_ERR_DEVICE
    assert qn(fp4, fp4.make_opts(fp4.FP4_NVFP4), batch=63, rows=8192, cols=8192) == fp4.FP4_ERR_DEVICE
    assert qn(fp4, fp4.make_opts(fp4.FP4_MXFP4)) == fp4.FP4_ERR_DEVICE


@cpu_only
def test_valid_quantize_without_gfx950_reports_device(fp4):
    assert q(fp4, fp4.make_opts(fp4.FP4_NVFP4)) == fp4.FP4_ERR_DEVICE
    assert q(fp4, fp4.make_opts(fp4.FP4_MXFP4), ws=0, ws_bytes=0) == fp4.FP4_ERR_DEVICE


def d(fp4, fmt=1, batch=1, rows=8, cols=64, codes=FAKE, ldc=32, scales=FAKE, lds=4, ts=FAKE, y=FAKE, yt=0, ldy=64,
      bsy=0):
    return fp4.fp4_dequantize(fmt, batch, rows, cols, codes, ldc, 0, scales, lds, 0, ts, y, yt, ldy, bsy, None)


def test_dequantize_errors(fp4):
    assert d(fp4, fmt=3) == fp4.FP4_ERR_INVALID
    assert d(fp4, yt=9) == fp4.FP4_ERR_INVALID
    assert d(fp4, cols=24, ldc=12, ldy=24) == fp4.FP4_ERR_INVALID
    assert d(fp4, fmt=0, cols=48, ldc=24, lds=2, ldy=48) == fp4.FP4_ERR_INVALID
    assert d(fp4, ts=0) == fp4.FP4_ERR_INVALID
    assert d(fp4, ldy=32) == fp4.FP4_ERR_INVALID
    assert d(fp4, batch=2, bsy=100) == fp4.FP4_ERR_INVALID
    assert d(fp4, y=FAKE + 4) == fp4.FP4_ERR_ALIGN
    assert d(fp4, codes=FAKE + 2) == fp4.FP4_ERR_ALIGN
    assert d(fp4, rows=0, codes=0, scales=0, ts=0, y=0) == fp4.FP4_OK


@cpu_only
def test_valid_dequantize_without_gfx950_reports_device(fp4):
    assert d(fp4) == fp4.FP4_ERR_DEVICE


def g(fp4, fmt=0, groups=1, M=64, N=64, K=128, a=FAKE, lda=64, ags=0, asc=FAKE, ldas=16, asgs=0, ats=FAKE, b=FAKE,
      ldb=64, bgs=0, bsc=FAKE, ldbs=16, bsgs=0, bts=FAKE, c=FAKE, ct=0, ldc=64, cgs=0):
    return fp4.fp4_gemm(fmt, groups, M, N, K, a, lda, ags, asc, ldas, asgs, ats, b, ldb, bgs, bsc, ldbs, bsgs, bts,
                        c, ct, ldc, cgs, None)


def test_gemm_errors(fp4):
    assert g(fp4, fmt=2) == fp4.FP4_ERR_INVALID
    assert g(fp4, ct=3) == fp4.FP4_ERR_INVALID
    assert g(fp4, K=96, lda=48, ldb=48, ldas=3, ldbs=3) == fp4.FP4_ERR_INVALID   # K % 64
    assert g(fp4, lda=32) == fp4.FP4_ERR_INVALID
    assert g(fp4, ldas=2) == fp4.FP4_ERR_INVALID
    assert g(fp4, ldc=32) == fp4.FP4_ERR_INVALID
    assert g(fp4, fmt=1, ats=0) == fp4.FP4_ERR_INVALID
    assert g(fp4, groups=2, ags=4096, bgs=4096, asgs=1024, bsgs=1024, cgs=100) == fp4.FP4_ERR_INVALID
    assert g(fp4, a=FAKE + 8) == fp4.FP4_ERR_ALIGN
    assert g(fp4, lda=72) == fp4.FP4_ERR_ALIGN
    assert g(fp4, c=FAKE + 2) == fp4.FP4_ERR_ALIGN
    # scale rows are read 16 bytes at a time
    assert g(fp4, asc=FAKE + 8) == fp4.FP4_ERR_ALIGN
    assert g(fp4, ldbs=24) == fp4.FP4_ERR_ALIGN
    assert g(fp4, groups=2, ags=4096, bgs=4096, asgs=1032, bsgs=1024, cgs=4096) == fp4.FP4_ERR_ALIGN
    assert g(fp4, M=0, a=0, b=0, c=0) == fp4.FP4_OK
    assert g(fp4, M=-1) == fp4.FP4_ERR_INVALID
    # panels past 2 GiB, and row pitches of 8 MiB or more, are not addressed
    assert g(fp4, M=1 << 16, lda=1 << 15) == fp4.FP4_ERR_UNSUPPORTED
    assert g(fp4, M=1, lda=1 << 23) == fp4.FP4_ERR_UNSUPPORTED
    assert g(fp4, N=1, ldbs=1 << 23) == fp4.FP4_ERR_UNSUPPORTED


@cpu_only
def test_valid_gemm_without_gfx950_reports_device(fp4):
    assert g(fp4) == fp4.FP4_ERR_DEVICE
    assert g(fp4, fmt=1) == fp4.FP4_ERR_DEVICE


def gq(fp4, opts, N=64, oc=FAKE, ldoc=32, os_=FAKE, ldos=16, ots=FAKE, groups=1, ocgs=0, osgs=0, **kw):
    """fp4_gemm_quantize_output with the operand arguments of g()."""
    a = dict(fmt=0, M=64, K=128, a=FAKE, lda=64, ags=0, asc=FAKE, ldas=16, asgs=0, ats=FAKE, b=FAKE, ldb=64, bgs=0,
             bsc=FAKE, ldbs=16, bsgs=0, bts=FAKE)
    a.update(kw)
    return fp4.fp4_gemm_quantize_output(a["fmt"], groups, a["M"], N, a["K"], a["a"], a["lda"], a["ags"], a["asc"],
                                        a["ldas"], a["asgs"], a["ats"], a["b"], a["ldb"], a["bgs"], a["bsc"],
                                        a["ldbs"], a["bsgs"], a["bts"], opts, oc, ldoc, ocgs, os_, ldos, osgs, ots,
                                        None)


def test_gemm_quantize_output_errors(fp4):
    mx = fp4.make_opts(fp4.FP4_MXFP4)
    nv_amax = fp4.make_opts(fp4.FP4_NVFP4, amax_in=FAKE)
    assert gq(fp4, fp4.make_opts(fp4.FP4_NVFP4)) == fp4.FP4_ERR_INVALID            # NVFP4 output needs amax_in
    assert gq(fp4, nv_amax, ots=0) == fp4.FP4_ERR_INVALID                          # and a tensor-scale output
    assert gq(fp4, mx, N=48, ldoc=24) == fp4.FP4_ERR_INVALID                       # N % 32
    assert gq(fp4, mx, ldoc=16) == fp4.FP4_ERR_INVALID                             # pitch < N / 2
    assert gq(fp4, mx, oc=FAKE + 4) == fp4.FP4_ERR_ALIGN
    assert gq(fp4, mx, ldoc=36) == fp4.FP4_ERR_ALIGN
    for f in (fp4.FP4_BLOCK2D, fp4.FP4_TRANSPOSE):
        assert gq(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=f, amax_in=FAKE)) == fp4.FP4_ERR_UNSUPPORTED
    assert gq(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=fp4.FP4_SCALE_SEARCH)) == fp4.FP4_ERR_UNSUPPORTED
    assert gq(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=128, amax_in=FAKE)) == fp4.FP4_ERR_INVALID
    assert gq(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=fp4.FP4_TENSOR_SCALE, amax_in=FAKE)) == fp4.FP4_ERR_UNSUPPORTED
    assert gq(fp4, mx, fmt=3) == fp4.FP4_ERR_INVALID                               # operand format
    assert gq(fp4, mx, M=0) == fp4.FP4_OK


@cpu_only
def test_valid_gemm_quantize_output_without_gfx950_reports_device(fp4):
    assert gq(fp4, fp4.make_opts(fp4.FP4_MXFP4, flags=fp4.FP4_FOUR_OVER_SIX)) == fp4.FP4_ERR_DEVICE
    assert gq(fp4, fp4.make_opts(fp4.FP4_NVFP4, flags=fp4.FP4_SCALE_SEARCH, amax_in=FAKE), fmt=1) == \
        fp4.FP4_ERR_DEVICE


def gg(fp4, groups=2, offs=FAKE, M=64, N=64, K=128, a=FAKE, lda=64, asc=FAKE, ldas=16, ats=FAKE, b=FAKE, ldb=64,
       bgs=4096, bsc=FAKE, ldbs=16, bsgs=1024, bts=FAKE, c=FAKE, ct=0, ldc=64, fmt=0):
    return fp4.fp4_gemm_grouped(fmt, groups, offs, M, N, K, a, lda, asc, ldas, ats, b, ldb, bgs, bsc, ldbs, bsgs,
                                bts, c, ct, ldc, None)


def test_gemm_grouped_errors(fp4):
    assert gg(fp4, offs=0) == fp4.FP4_ERR_INVALID
    assert gg(fp4, offs=FAKE + 2) == fp4.FP4_ERR_ALIGN
    assert gg(fp4, groups=5000) == fp4.FP4_ERR_UNSUPPORTED
    assert gg(fp4, K=96, lda=48, ldb=48, ldas=3, ldbs=3) == fp4.FP4_ERR_INVALID
    assert gg(fp4, ldc=32) == fp4.FP4_ERR_INVALID
    assert gg(fp4, fmt=1, ats=0) == fp4.FP4_ERR_INVALID
    assert gg(fp4, bgs=4104) == fp4.FP4_ERR_ALIGN
    assert gg(fp4, groups=0, offs=0) == fp4.FP4_OK
    assert gg(fp4, M=0) == fp4.FP4_OK


@cpu_only
def test_valid_gemm_grouped_without_gfx950_reports_device(fp4):
    assert gg(fp4) == fp4.FP4_ERR_DEVICE


def test_product_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_scaled_fp4_amax_amd as F
    monkeypatch.setattr(F, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(F, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        F.lib()
