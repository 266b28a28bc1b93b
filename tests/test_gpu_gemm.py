"""GPU parity of fp4_gemm against the oracle's reference, the pages' FP32
fallback: dequantize both operands, then matmul (here in float64). The GEMM's
operands are the oracle's own codes and scales, uploaded, so nothing on the
reference side comes from the HIP path.

Tolerance (fp32 output): relative Frobenius error <= 1e-3, and element-wise
|C - C_ref| <= (2K + 4) * 2^-24 * (|A| |B|^T) (fp32 accumulation over K plus
the epilogue scaling). bf16 output: the same plus one bf16 rounding,
2^-8 * |C_ref|."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as F
from block_scaled_fp4_amax_amd import inputs
from gpu_util import check_close, flag_str, oracle_operand

pytestmark = pytest.mark.gpu

MX, NV = 0, 1
FOS, B2D, TR, SR, RHT = 1, 2, 4, 8, 16


def run_case(O, a, b, fmt, fa, fb, out_dtype, signs=0, what=""):
    print(f"[gemm] {what} fmt={fmt} A{tuple(a.shape)} {flag_str(fa)} B{tuple(b.shape)} {flag_str(fb)} -> {out_dtype}",
          flush=True)
    qa, da = oracle_operand(O, a, fmt, fa, signs)
    qb, db = oracle_operand(O, b, fmt, fb, signs)
    c = F.gemm(qa, qb, out_dtype)
    torch.cuda.synchronize()
    c3 = c if c.dim() == 3 else c.unsqueeze(0)
    for g in range(da.shape[0]):
        ref = O.gemm_reference(da[g], db[g])
        absab = np.abs(da[g]).astype(np.float64) @ np.abs(db[g]).astype(np.float64).T
        check_close(c3[g], ref, absab, da.shape[-1], out_dtype, f"{what} group {g}")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_mxfp4_dense_ragged(oracle, out):
    a = inputs.w4a4_linear(m=70, n=200, k=320)
    run_case(oracle, a["a"], a["w"], MX, 0, 0, out, what="mx-dense")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_mxfp4_grouped_moe_recipe(oracle, out):
    d = inputs.moe_mxfp4(experts=3, tokens=40, k=2880, n=96)
    run_case(oracle, d["x"], d["w"], MX, 0, TR, out, what="mx-grouped")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("flags", [0, FOS])
def test_nvfp4_dense_ragged(oracle, out, flags):
    d = inputs.w4a4_linear(m=200, n=272, k=320)
    run_case(oracle, d["a"], d["w"], NV, flags, flags, out, what="nv-dense")


@pytest.mark.parametrize("k", [64, 128, 192, 384, 576, 1088, 2112])
@pytest.mark.parametrize("fmt", [MX, NV], ids=["mx", "nv"])
def test_k_pipeline_depths(oracle, fmt, k):
    """K from one half-stage (64) up to several rounds of the 4-slot stage
    ring, with and without a final half-stage, and scale chunks that end
    part-way through a stage group."""
    d = inputs.w4a4_linear(m=40, n=72, k=k, seed=k)
    run_case(oracle, d["a"], d["w"], fmt, FOS if fmt == NV else 0, FOS if fmt == NV else 0, torch.float32,
             what=f"k-sweep K={k}")


@pytest.mark.parametrize("fmt", [MX, NV], ids=["mx", "nv"])
def test_every_block_scale_code(oracle, fmt):
    """Random codes under block scales that run through every finite E4M3
    code, zero and the subnormals included (NVFP4), or through 2^-17 .. 2^17
    (MXFP4), on both operands, against the oracle's dequantize-then-matmul.
    The codes and scales are set directly, not quantized."""
    from gpu_util import upload_scales
    rng = np.random.default_rng(11 + fmt)
    M, N, K = 127, 96, 512
    blk = 16 if fmt == NV else 32
    ca = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    cb = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    if fmt == NV:
        # 37 and 53 are prime to 127: each code appears about equally often
        sa = (np.arange(M * (K // blk)) * 37 % 127).astype(np.uint8).reshape(M, K // blk)
        sb = (np.arange(N * (K // blk)) * 53 % 127).astype(np.uint8).reshape(N, K // blk)
        ts_a, ts_b = 0.125, 4.0
    else:
        sa = (110 + np.arange(M * (K // blk)) * 3 % 35).astype(np.uint8).reshape(M, K // blk)
        sb = (110 + np.arange(N * (K // blk)) * 5 % 35).astype(np.uint8).reshape(N, K // blk)
        ts_a = ts_b = None
    da = oracle.dequantize(fmt, ca, sa, ts_a)
    db = oracle.dequantize(fmt, cb, sb, ts_b)

    def upload(codes, scales, ts):
        t = torch.tensor([ts], dtype=torch.float32).cuda() if ts is not None else None
        return F.Quantized(fmt, torch.from_numpy(codes).cuda(), upload_scales(scales), t)

    print(f"[gemm] every-scale-code fmt={fmt} {M}x{N}x{K}", flush=True)
    c = F.gemm(upload(ca, sa, ts_a), upload(cb, sb, ts_b), torch.float32)
    torch.cuda.synchronize()
    c = c if c.dim() == 2 else c[0]
    ref = oracle.gemm_reference(da, db)
    absab = np.abs(da).astype(np.float64) @ np.abs(db).astype(np.float64).T
    check_close(c, ref, absab, K, torch.float32, f"every-scale-code fmt={fmt}")


def test_nvfp4_grouped(oracle):
    a = torch.stack([inputs.w4a4_linear(m=33, n=64, k=128, seed=s)["a"] for s in range(3)])
    b = torch.stack([inputs.w4a4_linear(m=33, n=64, k=128, seed=s)["w"] for s in range(3)])
    run_case(oracle, a, b, NV, FOS, FOS, torch.float32, what="nv-grouped")


def test_nvfp4_rht_recipe(oracle):
    d = inputs.rht_activation(m=100, k=256, n=160)
    run_case(oracle, d["x"], d["w"], NV, FOS | RHT, FOS | RHT | TR, torch.float32, signs=d["signs"], what="nv-rht")


def test_rht_cancels_in_the_product(oracle):
    """Same sign mask on both operands: the rotated FP4 product approximates
    the unrotated bf16 product about as well as plain FP4 does."""
    d = inputs.rht_activation(m=128, k=512, n=256)
    exact = d["x"].double() @ d["w"].double()
    qa, _ = oracle_operand(oracle, d["x"], NV, FOS | RHT, d["signs"])
    qb, _ = oracle_operand(oracle, d["w"], NV, FOS | RHT | TR, d["signs"])
    c = F.gemm(qa, qb, torch.float32).double().cpu()[0]
    rel = (c - exact).norm() / exact.norm()
    assert rel < 0.2, rel


# ---------------------------------------------------------------------------
# full sizes (the benchmark's launch configurations), sampled outputs
# ---------------------------------------------------------------------------
def full_case(O, a, b, fmt, fa, fb, signs=0, what=""):
    """The product at full size, written as bf16 and as fp32 (the 1e-3
    relative Frobenius bound applies to the fp32 output, here on 48 x 48
    sampled outputs of up to three groups)."""
    print(f"[gemm-full] {what} A{tuple(a.shape)} B{tuple(b.shape)}", flush=True)
    a3 = a.unsqueeze(0) if a.dim() == 2 else a
    b3 = b.unsqueeze(0) if b.dim() == 2 else b
    G = a3.shape[0]
    M = a3.shape[1]
    N = b3.shape[2] if fb & TR else b3.shape[1]
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(M, size=min(M, 48), replace=False))
    cols = np.sort(rng.choice(N, size=min(N, 48), replace=False))
    qa, da = oracle_operand(O, a3.cpu(), fmt, fa, signs, rows=rows)
    qb, db = oracle_operand(O, b3.cpu(), fmt, fb, signs, rows=cols)
    groups = sorted(set(rng.integers(0, G, 3).tolist()))
    for out_dtype in (torch.bfloat16, torch.float32):
        print(f"[gemm-full] {what} -> {out_dtype}", flush=True)
        c = F.gemm(qa, qb, out_dtype)
        torch.cuda.synchronize()
        c3 = c if c.dim() == 3 else c.unsqueeze(0)
        for g in groups:
            ref = O.gemm_reference(da[g], db[g])
            absab = np.abs(da[g]).astype(np.float64) @ np.abs(db[g]).astype(np.float64).T
            got = c3[g][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
            check_close(got, ref, absab, da.shape[-1], out_dtype, f"{what} {out_dtype} group {g}")
        del c, c3


def test_full_w4a4_linear(oracle):
    d = inputs.w4a4_linear(device="cuda")
    full_case(oracle, d["a"], d["w"], NV, FOS, FOS, what="2048x4096x4096 nvfp4")


def test_full_moe_grouped(oracle):
    d = inputs.moe_mxfp4(device="cuda")
    full_case(oracle, d["x"], d["w"], MX, 0, TR, what="32x512x5760x2880 mxfp4")


def test_full_rht_gemm(oracle):
    d = inputs.rht_activation(device="cuda")
    full_case(oracle, d["x"], d["w"], NV, FOS | RHT, FOS | RHT | TR, signs=d["signs"],
              what="16384x12288x4096 nvfp4 rht")


def test_nvfp4_wide_tile_ragged(oracle):
    """The 256-wide NVFP4 tile (enough tiles for every compute unit and a long
    K): 4100 x 3900 x 2112 leaves a partial last M tile (4 rows) and N tile
    (60 columns), and K = 33 half-stages ends on a half stage. Sampled outputs
    include the first and last rows and columns of every partial tile."""
    d = inputs.w4a4_linear(m=4100, n=3900, k=2112, device="cuda")
    a, b = d["a"].unsqueeze(0), d["w"].unsqueeze(0)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(4100, 40, replace=False), [0, 255, 256, 4095, 4096, 4099]]))
    cols = np.unique(np.concatenate([rng.choice(3900, 40, replace=False), [0, 255, 256, 3839, 3840, 3899]]))
    qa, da = oracle_operand(oracle, a.cpu(), NV, FOS, rows=rows)
    qb, db = oracle_operand(oracle, b.cpu(), NV, FOS, rows=cols)
    ref = oracle.gemm_reference(da[0], db[0])
    absab = np.abs(da[0]).astype(np.float64) @ np.abs(db[0]).astype(np.float64).T
    for out_dtype in (torch.bfloat16, torch.float32):
        print(f"[gemm-wide] 4100x3900x2112 nvfp4 -> {out_dtype}", flush=True)
        c = F.gemm(qa, qb, out_dtype)
        torch.cuda.synchronize()
        assert tuple(c.shape) == (1, 4100, 3900), c.shape
        got = c[0][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
        check_close(got, ref, absab, da.shape[-1], out_dtype, f"wide nvfp4 {out_dtype}")
