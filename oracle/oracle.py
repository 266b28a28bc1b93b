"""Python wrapper of the CPU oracle (``fp4_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library. It shares no
code with the HIP path.

Every function below follows the C oracle; the C file states, step by step,
the passage of the pages each part follows and every reading taken where the
pages are silent. Pins (tests/test_oracle_pins.py) tie each part to something
other than the oracle itself:

  E2M1 grid / RNE      the pages' 15-value grid; brute-force nearest search
  worked example       the pages' printed MAE 0.7238 / 0.0901 / 0.0747
  E4M3 encode/decode   torch.float8_e4m3fn (exhaustive over [0, 448])
  E8M0 exponent        math.frexp closed form; torch.float8_e8m0fnu decode
  Philox4x32-10        rocRAND's independent implementation
  stochastic rounding  unbiasedness on exact fractions; brute-force bracket
  Hadamard transform   dense Sylvester matrix (exact rational), orthogonality
  MXFP4 / NVFP4 / 4/6  exact argmin of the candidates' errors on 10^5 blocks
  and the scale search   each (float64 certified to 1e-13, spot-checked with
                       fractions), outside a band derived from the float32
                       evaluation the readings fix; exact nearest E4M3 and
                       E2M1 codes outside their rounding bands; invariants
                       (saturation, scale 448)
  RHT and SR inside    quantize with the transform = quantize of the exactly
  the quantizer        rotated copy; every SR code = e2m1_sr of the scaled
                       value with rocRAND's draw of its output index;
                       unbiased mean over 2^12 offsets
  2D / transpose       transpose symmetry, constant tiles reduce to 1D
  GEMM reference       dequantize + numpy float64 matmul (library routine)
  grouped GEMM         brute-force sum over k per output element; one group
                       equals the plain product

Parity of the MXFP4 / NVFP4 / 4-over-6 MAE values on the worked example is
unpinned by the pages (they print only the float-scale numbers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import c_float, c_int, c_int32, c_int64, c_uint8, c_uint32, c_uint64, c_void_p
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "fp4_oracle.c"
LIB = HERE / "liboracle.so"

MXFP4, NVFP4 = 0, 1
F32, BF16 = 0, 1
FOUR_OVER_SIX, BLOCK2D, TRANSPOSE, STOCHASTIC, HADAMARD, SCALE_SEARCH, TENSOR_SCALE = 1, 2, 4, 8, 16, 32, 64

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build() -> Path:
    cmd = ["gcc", *CFLAGS, str(SRC), "-o", str(LIB) + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(str(LIB) + ".tmp", LIB)
    return LIB


class _Opts(ctypes.Structure):
    _fields_ = [("format", c_int), ("flags", ctypes.c_uint), ("seed", c_uint64), ("offset", c_uint64),
                ("rht_signs", c_uint32), ("has_amax", c_int), ("amax", c_float)]


_L = None


def lib():
    global _L
    if _L is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        L = ctypes.CDLL(str(LIB))
        L.or_e2m1_value.restype = c_float
        L.or_e2m1_value.argtypes = [c_uint8]
        L.or_e2m1_rne.restype = c_uint8
        L.or_e2m1_rne.argtypes = [c_float]
        L.or_e2m1_sr.restype = c_uint8
        L.or_e2m1_sr.argtypes = [c_float, c_uint32]
        L.or_e4m3_value.restype = c_float
        L.or_e4m3_value.argtypes = [c_uint8]
        L.or_e4m3_rne.restype = c_uint8
        L.or_e4m3_rne.argtypes = [c_float]
        L.or_e8m0_exponent.restype = c_int
        L.or_e8m0_exponent.argtypes = [c_float]
        L.or_philox4x32_10.restype = None
        L.or_philox4x32_10.argtypes = [c_void_p, c_void_p, c_void_p]
        L.or_sr_random16.restype = c_uint32
        L.or_sr_random16.argtypes = [c_uint64, c_uint64, c_uint64]
        L.or_rht16.restype = None
        L.or_rht16.argtypes = [c_void_p, c_uint32]
        L.or_tensor_amax.restype = c_float
        L.or_tensor_amax.argtypes = [c_void_p, c_int, c_int64, c_int64, c_int64, ctypes.c_uint, c_uint32]
        L.or_nvfp4_tensor_scale.restype = c_float
        L.or_nvfp4_tensor_scale.argtypes = [c_float, c_int]
        L.or_quantize.restype = c_int
        L.or_quantize.argtypes = [c_void_p, c_int, c_int64, c_int64, c_int64, ctypes.POINTER(_Opts), c_uint64,
                                  c_void_p, c_void_p, c_void_p, c_void_p]
        L.or_dequantize.restype = c_int
        L.or_dequantize.argtypes = [c_int, c_int64, c_int64, c_void_p, c_void_p, c_float, c_void_p]
        L.or_float_scale_dequant.restype = c_int
        L.or_float_scale_dequant.argtypes = [c_void_p, c_int64, c_int64, c_void_p]
        for nm in ("or_e2m1_rne_n", "or_e4m3_rne_n"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [c_void_p, c_int64, c_void_p]
        L.or_e2m1_sr_n.restype = None
        L.or_e2m1_sr_n.argtypes = [c_void_p, c_void_p, c_int64, c_void_p]
        L.or_e8m0_exponent_n.restype = None
        L.or_e8m0_exponent_n.argtypes = [c_void_p, c_int64, c_void_p]
        _L = L
    return _L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(c_void_p)


# --- element codecs ---------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(code)


def e2m1_rne(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(-1)
    out = np.empty(q.size, np.uint8)
    lib().or_e2m1_rne_n(_ptr(q), q.size, _ptr(out))
    return out


def e2m1_sr(q, r16) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(-1)
    r = np.ascontiguousarray(r16, dtype=np.uint32).reshape(-1)
    out = np.empty(q.size, np.uint8)
    lib().or_e2m1_sr_n(_ptr(q), _ptr(r), q.size, _ptr(out))
    return out


def e4m3_value(code: int) -> float:
    return lib().or_e4m3_value(code)


def e4m3_rne(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32).reshape(-1)
    out = np.empty(s.size, np.uint8)
    lib().or_e4m3_rne_n(_ptr(s), s.size, _ptr(out))
    return out


def e8m0_exponent(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    out = np.empty(a.size, np.int32)
    lib().or_e8m0_exponent_n(_ptr(a), a.size, _ptr(out))
    return out


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_random16(seed: int, offset: int, L: int) -> int:
    return lib().or_sr_random16(seed, offset, L)


def rht16(v, signs: int) -> np.ndarray:
    a = np.array(v, dtype=np.float32).reshape(16).copy()
    lib().or_rht16(_ptr(a), signs)
    return a


def nvfp4_tensor_scale(amax: float, four_over_six: bool, whole_tensor: bool = False) -> float:
    return lib().or_nvfp4_tensor_scale(amax, 2 if whole_tensor else int(bool(four_over_six)))


# --- tensors ----------------------------------------------------------------
def _as_input(x: np.ndarray):
    """x: float32 array, or uint16 array of bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")


def tensor_amax(x: np.ndarray, flags: int = 0, rht_signs: int = 0) -> float:
    x, dt = _as_input(x)
    rows, cols = x.shape
    return lib().or_tensor_amax(_ptr(x), dt, rows, cols, cols, flags, rht_signs)


def quantize(x: np.ndarray, fmt: int, flags: int = 0, rht_signs: int = 0, seed: int = 0, offset: int = 0,
             amax: float | None = None, L0: int = 0) -> dict:
    """Quantize one matrix [rows, cols]. Returns dict(codes, scales,
    tensor_scale, amax); codes [R, C/2] uint8, scales [R, C/blk] uint8."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    tr = bool(flags & TRANSPOSE)
    R, C = (cols, rows) if tr else (rows, cols)
    blk = 16 if fmt == NVFP4 else 32
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // blk), np.uint8)
    ts = np.zeros(1, np.float32)
    am = np.zeros(1, np.float32)
    o = _Opts(fmt, flags, seed, offset, rht_signs, int(amax is not None), float(amax or 0.0))
    rc = lib().or_quantize(_ptr(x), dt, rows, cols, cols, ctypes.byref(o), L0, _ptr(codes), _ptr(scales), _ptr(ts),
                           _ptr(am))
    if rc != 0:
        raise ValueError("oracle: shape/options not defined")
    return {"codes": codes, "scales": scales, "tensor_scale": float(ts[0]) if fmt == NVFP4 else None,
            "amax": float(am[0]) if fmt == NVFP4 else None}


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, tensor_scale: float | None = None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    R, half = codes.shape
    y = np.empty((R, half * 2), np.float32)
    rc = lib().or_dequantize(fmt, R, half * 2, _ptr(codes), _ptr(scales), float(tensor_scale or 0.0), _ptr(y))
    if rc != 0:
        raise ValueError("oracle: bad dequantize shape")
    return y


def float_scale_dequant(x: np.ndarray, block: int) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).reshape(-1)
    y = np.empty_like(x)
    if lib().or_float_scale_dequant(_ptr(x), x.size, block, _ptr(y)) != 0:
        raise ValueError("bad block")
    return y


def gemm_reference(a_deq: np.ndarray, b_deq: np.ndarray) -> np.ndarray:
    """The pages' FP32-simulated matmul fallback, evaluated in float64:
    C = deq(A) @ deq(B)^T."""
    return np.asarray(a_deq, np.float64) @ np.asarray(b_deq, np.float64).T


def grouped_gemm_reference(a_deq: np.ndarray, b_deq: np.ndarray, offsets) -> np.ndarray:
    """The mixture-of-experts grouped product: rows offsets[g]:offsets[g+1]
    of deq(A) [M, K] times deq(B_g)^T, B [G, N, K]; rows outside every group
    stay NaN (not written). offsets: nondecreasing, G + 1 entries."""
    a = np.asarray(a_deq, np.float64)
    b = np.asarray(b_deq, np.float64)
    c = np.full((a.shape[0], b.shape[1]), np.nan)
    for g in range(b.shape[0]):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        c[lo:hi] = gemm_reference(a[lo:hi], b[g])
    return c
