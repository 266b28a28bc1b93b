"""GPU parity of fp4_gemm_quantize_output: the W4A4 GEMM whose epilogue
quantizes the product along its rows (MXFP4 or NVFP4, with 4/6, stochastic
rounding and the Hadamard transform as options) instead of storing it.

Bit-exact parity with the oracle needs the oracle's product to be the
kernel's fp32 product. The first test builds operands whose dequantized
values all have few significant bits within a narrow exponent range and
whose tensor scales are powers of two, checks (in float64) that every
partial sum of the product is then exact in fp32, and requires codes,
scales and tensor scales equal to the oracle's quantization of its own
product. On general inputs the kernel must produce exactly what the
unfused path produces (fp4_gemm to fp32, then fp4_quantize), and at the
benchmark's size the dequantized output must lie within the rounding error
of the oracle's product."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as F
from block_scaled_fp4_amax_amd import inputs
from gpu_util import assert_codes_equal, flag_str, oracle_operand, oracle_quantize

pytestmark = pytest.mark.gpu

MX, NV = 0, 1
FOS, SR, RHT, SEARCH = 1, 8, 16, 32
SIGNS = 0xA5C3
SEED, OFFSET = 21, 5

# (operand format, operand flags, output format, output flags)
CASES = [(MX, 0, MX, 0), (MX, 0, MX, SR), (MX, 0, MX, RHT), (NV, FOS, MX, SR | RHT),
         (NV, 0, NV, 0), (NV, FOS, NV, FOS), (NV, FOS, NV, SR), (NV, FOS, NV, FOS | SR),
         (MX, 0, NV, FOS | RHT), (NV, FOS, NV, FOS | SR | RHT), (MX, 0, MX, FOS), (NV, FOS, MX, FOS | SR),
         (NV, FOS, NV, SEARCH), (MX, 0, NV, SEARCH | SR | RHT)]
IDS = [f"{'nv' if a == NV else 'mx'}-{flag_str(fa)}->{'nv' if o == NV else 'mx'}-{flag_str(fo)}"
       for a, fa, o, fo in CASES]

GRID = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0])


def structured(G, rows, cols, blk, peak, seed):
    """E2M1 grid values with random signs, each block scaled by 2^0 or 2^-1
    with its first element at the block's largest grid value, and one
    element equal to `peak` (which fixes the NVFP4 tensor scale: 10.5 / 2688
    = 7 / 1792 = 2^-8)."""
    rng = np.random.default_rng(seed)
    x = rng.choice(GRID, size=(G, rows, cols)) * rng.choice([-1.0, 1.0], size=(G, rows, cols))
    e = np.repeat(2.0 ** rng.integers(-1, 1, size=(G, rows, cols // blk)), blk, axis=2)
    x = x * e
    x[:, :, ::blk] = 6.0 * e[:, :, ::blk] * np.sign(x[:, :, ::blk])
    for g in range(G):
        x[g, rng.integers(rows), rng.integers(cols)] = peak
    return torch.from_numpy(x.astype(np.float32))


def lsb_exponent(v):
    """Smallest exponent of a set bit over the nonzero values of v."""
    v = np.abs(v[v != 0]).astype(np.float64)
    m, e = np.frexp(v)
    mi = (m * 2.0 ** 53).astype(np.int64)
    return int((e - 53 + np.log2((mi & -mi).astype(np.float64)).astype(np.int64)).min())


def run_fused(qa, qb, fo_fmt, fo, amax):
    return F.gemm_quantize_output(qa, qb, "nvfp4" if fo_fmt == NV else "mxfp4", four_over_six=bool(fo & FOS),
                                  stochastic=bool(fo & SR), hadamard=bool(fo & RHT), scale_search=bool(fo & SEARCH),
                                  rht_signs=SIGNS, seed=SEED, offset=OFFSET, amax=amax)


def compare(got, codes, scales, ts, fo_fmt, what):
    torch.cuda.synchronize()
    gc = got.codes.cpu().numpy()
    gs = got.scales.cpu().numpy()
    assert_codes_equal(gc, codes, f"{what} codes")
    assert_codes_equal(gs, scales, f"{what} scales")
    if fo_fmt == NV:
        assert np.array_equal(got.tensor_scale.cpu().numpy(), ts), f"{what} tensor scales"


@pytest.mark.parametrize("fa_fmt,fa,fo_fmt,fo", CASES, ids=IDS)
def test_exact_product_matches_oracle(oracle, fa_fmt, fa, fo_fmt, fo):
    print(f"[fused] exact {fa_fmt},{flag_str(fa)} -> {fo_fmt},{flag_str(fo)}", flush=True)
    blk = 16 if fa_fmt == NV else 32
    G, M, N, K = 2, 96, 160, 256
    peak = 7.0 if fa & FOS else 10.5
    qa, da = oracle_operand(oracle, structured(G, M, K, blk, peak, 1), fa_fmt, fa)
    qb, db = oracle_operand(oracle, structured(G, N, K, blk, peak, 2), fa_fmt, fa)
    c = np.stack([oracle.gemm_reference(da[g], db[g]) for g in range(G)])
    absab = np.stack([np.abs(da[g]).astype(np.float64) @ np.abs(db[g]).astype(np.float64).T for g in range(G)])
    # every partial sum is a multiple of 2^q below 2^(24 + q): exact in fp32
    q = lsb_exponent(da) + lsb_exponent(db)
    assert absab.max() < 2.0 ** (24 + q)
    c32 = c.astype(np.float32)
    assert np.array_equal(c32.astype(np.float64), c)
    amax = np.abs(c32).reshape(G, -1).max(axis=1) if fo_fmt == NV else None
    codes, scales, ts = oracle_quantize(oracle, torch.from_numpy(c32), fo_fmt, fo, SIGNS, SEED, OFFSET, amax)
    got = run_fused(qa, qb, fo_fmt, fo, torch.from_numpy(amax).cuda() if amax is not None else None)
    compare(got, codes, scales, ts, fo_fmt, "exact")


def test_exact_product_saturating_amax(oracle):
    """NVFP4 output with a supplied amax below the true one: blocks above it
    saturate exactly as fp4_quantize saturates them."""
    G, M, N, K = 1, 64, 96, 128
    qa, da = oracle_operand(oracle, structured(G, M, K, 16, 10.5, 3), NV, 0)
    qb, db = oracle_operand(oracle, structured(G, N, K, 16, 10.5, 4), NV, 0)
    c32 = oracle.gemm_reference(da[0], db[0]).astype(np.float32)[None]
    amax = np.array([0.25 * np.abs(c32).max()], np.float32)
    codes, scales, ts = oracle_quantize(oracle, torch.from_numpy(c32), NV, FOS, 0, 0, 0, amax)
    got = F.gemm_quantize_output(qa, qb, "nvfp4", four_over_six=True, amax=torch.from_numpy(amax).cuda())
    compare(got, codes, scales, ts, NV, "saturating")


@pytest.mark.parametrize("fa_fmt,fa,fo_fmt,fo", CASES, ids=IDS)
def test_matches_unfused_path(oracle, fa_fmt, fa, fo_fmt, fo):
    """General inputs: the fused epilogue equals fp4_gemm (fp32) followed by
    fp4_quantize of its output, bit for bit."""
    print(f"[fused] unfused {fa_fmt},{flag_str(fa)} -> {fo_fmt},{flag_str(fo)}", flush=True)
    d = inputs.w4a4_linear(m=200, n=288, k=320, seed=8)
    a = torch.stack([d["a"], (d["a"].float() * 0.5).to(torch.bfloat16)])
    b = torch.stack([d["w"], d["w"]])
    qa, _ = oracle_operand(oracle, a, fa_fmt, fa)
    qb, _ = oracle_operand(oracle, b, fa_fmt, fa)
    c = F.gemm(qa, qb, torch.float32)
    amax = c.abs().reshape(2, -1).amax(dim=1) if fo_fmt == NV else None
    ref = F.quantize(c, "nvfp4" if fo_fmt == NV else "mxfp4", four_over_six=bool(fo & FOS),
                     stochastic=bool(fo & SR), hadamard=bool(fo & RHT), scale_search=bool(fo & SEARCH),
                     rht_signs=SIGNS, seed=SEED, offset=OFFSET, amax=amax)
    got = run_fused(qa, qb, fo_fmt, fo, amax)
    torch.cuda.synchronize()
    compare(got, ref.codes.cpu().numpy(), ref.scales.cpu().numpy(),
            ref.tensor_scale.cpu().numpy() if ref.tensor_scale is not None else None, fo_fmt, "unfused")


def test_full_w4a4_fused(oracle):
    """The benchmark's launch: W4A4 2048 x 4096 x 4096 NVFP4 4/6 operands,
    NVFP4 4/6 output with its amax supplied. All of it against the unfused
    path; 32 sampled rows against the oracle's product: every dequantized
    output within one rounding step (2 eff) plus the GEMM's bound of it."""
    d = inputs.w4a4_linear(device="cuda")
    print("[fused-full] 2048x4096x4096", flush=True)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(2048, size=32, replace=False))
    qa, da = oracle_operand(oracle, d["a"].cpu(), NV, FOS, rows=rows)
    qb, db = oracle_operand(oracle, d["w"].cpu(), NV, FOS)
    c = F.gemm(qa, qb, torch.float32)
    amax = c.abs().amax().reshape(1)
    ref = F.quantize(c[0], "nvfp4", four_over_six=True, amax=amax)
    got = F.gemm_quantize_output(qa, qb, "nvfp4", four_over_six=True, amax=amax)
    torch.cuda.synchronize()
    compare(got, ref.codes[None].cpu().numpy(), ref.scales[None].cpu().numpy(), ref.tensor_scale.cpu().numpy(), NV,
            "full unfused")
    cref = oracle.gemm_reference(da[0], db[0])
    absab = np.abs(da[0]).astype(np.float64) @ np.abs(db[0]).astype(np.float64).T
    codes = got.codes.cpu().numpy()[0][rows]
    scales = got.scales.cpu().numpy()[0][rows]
    ts = float(got.tensor_scale.cpu()[0])
    deq = oracle.dequantize(NV, codes, scales, ts).astype(np.float64)
    eff = np.repeat(np.array([[oracle.e4m3_value(int(s)) for s in r] for r in scales]) * ts, 16, axis=1)
    bound = 2.0 * eff + (2 * 4096 + 4) * 2.0 ** -24 * absab
    assert (np.abs(deq - cref) <= bound).all()
