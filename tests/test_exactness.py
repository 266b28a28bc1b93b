"""The format facts that make the NVFP4 GEMM's fp16 dequantization exact,
checked over every code: each finite E4M3 scale is a normal fp16, and each
E2M1 value times each E4M3 scale is itself an fp16 value, normal and inside
[2^-10, 2688]. So converting codes and scales to fp16 and multiplying them in
fp16 loses nothing (format definitions: Ultralytics glossary "FP4", section
"Como funciona FP4")."""
import numpy as np


def test_e4m3_scales_are_normal_fp16(oracle):
    for code in range(0x7F):  # 0x7F is the E4M3 NaN; scales never take it
        s = oracle.e4m3_value(code)
        h = np.float16(s)
        assert float(h) == s, code
        assert s == 0.0 or abs(s) >= np.finfo(np.float16).tiny, code


def test_e2m1_times_e4m3_is_exact_in_fp16(oracle):
    mags = sorted({abs(oracle.e2m1_value(c)) for c in range(16)} - {0.0})
    assert mags == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    lo, hi = np.inf, 0.0
    for code in range(1, 0x7F):
        s = oracle.e4m3_value(code)
        for v in mags:
            p = v * s  # exact in float64
            assert float(np.float16(p)) == p, (code, v)
            lo, hi = min(lo, p), max(hi, p)
    assert lo == 2.0 ** -10 and hi == 2688.0
    assert lo >= np.finfo(np.float16).tiny
