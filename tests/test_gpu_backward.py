"""GPU parity of the backward pass of a quantized linear Y = X W^T, run as
the product runs it: fp4_quantize of each operand, then fp4_gemm.

  dgrad  dX = Q(dY) . Q(W^T)^T      A = dY [M, N] quantized along N (stochastic
                                    rounding), B = W^T [K, N]: W [N, K] quantized
                                    transposed with 16x16 scales
  wgrad  dW = Q(dY^T) . Q(X^T)^T    A = dY^T [N, M] (transposed, stochastic),
                                    B = X^T [K, M] (transposed)

(Four Over Six, "Training"; the NVFP4 training recipe: 2D weight scales so the
forward and backward passes see the same weight values, stochastic rounding on
gradients.) Every quantized operand must equal the oracle's bit for bit, and
each product must match the oracle's dequantize-then-matmul reference within
the same bounds as the GEMM's own tests."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as F
from block_scaled_fp4_amax_amd import inputs
from gpu_util import assert_codes_equal, check_close, gpu_quantize, oracle_quantize

pytestmark = pytest.mark.gpu

NV = 1
FOS, B2D, TR, SR = 1, 2, 4, 8
SEED = 6
G_OFFSET, GT_OFFSET = 0, 1 << 40  # distinct Philox streams for the two quantizations of dY


def operand(O, x, flags, offset=0, rows=None):
    """Quantize x on the GPU and in the oracle; the two must agree bit for bit
    (on the output rows `rows` when given). Returns the GPU Quantized and the
    oracle's dequantized rows."""
    q, codes, scales, ts = gpu_quantize(F, x.cuda(), NV, flags, seed=SEED, offset=offset)
    oc, osc, ots = oracle_quantize(O, x.cpu(), NV, flags, seed=SEED, offset=offset)
    sel = slice(None) if rows is None else rows
    what = f"flags={flags} offset={offset}"
    assert_codes_equal(codes[0][sel], oc[0][sel], f"codes {what}")
    assert_codes_equal(scales[0][sel], osc[0][sel], f"scales {what}")
    assert ts[0] == ots[0], f"tensor scale {what}"
    return q, O.dequantize(NV, oc[0][sel], osc[0][sel], float(ots[0]))


def check_product(O, c, da, db, out_dtype, what, rows=None, cols=None):
    c = c if c.dim() == 2 else c[0]
    if rows is not None:
        c = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    ref = O.gemm_reference(da, db)
    absab = np.abs(da).astype(np.float64) @ np.abs(db).astype(np.float64).T
    check_close(c, ref, absab, da.shape[-1], out_dtype, what)


SHAPES = [(192, 320, 208), (64, 128, 48), (320, 192, 400)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_dgrad(oracle, m, n, k, out):
    print(f"[backward] dgrad M={m} N={n} K={k} -> {out}", flush=True)
    d = inputs.training_backward(m=m, n=n, k=k, seed=m + n + k)
    qg, dg = operand(oracle, d["grad"], FOS | SR, G_OFFSET)
    qwt, dwt = operand(oracle, d["w"], FOS | B2D | TR)
    dx = F.gemm(qg, qwt, out)
    torch.cuda.synchronize()
    assert tuple(dx.shape[-2:]) == (m, k)
    check_product(oracle, dx, dg, dwt, out, f"dgrad {m}x{n}x{k}")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_wgrad(oracle, m, n, k, out):
    print(f"[backward] wgrad M={m} N={n} K={k} -> {out}", flush=True)
    d = inputs.training_backward(m=m, n=n, k=k, seed=m + n + k)
    qgt, dgt = operand(oracle, d["grad"], FOS | SR | TR, GT_OFFSET)
    qxt, dxt = operand(oracle, d["x"], FOS | TR)
    dw = F.gemm(qgt, qxt, out)
    torch.cuda.synchronize()
    assert tuple(dw.shape[-2:]) == (n, k)
    check_product(oracle, dw, dgt, dxt, out, f"wgrad {m}x{n}x{k}")


def test_backward_weight_matches_forward_weight(oracle):
    """With 16x16 scales the weight the backward pass multiplies by (W
    quantized transposed) holds exactly the values of the forward pass's
    quantized W, transposed."""
    d = inputs.training_backward(m=64, n=256, k=192, seed=3)
    _, codes_f, scales_f, ts_f = gpu_quantize(F, d["w"].cuda(), NV, FOS | B2D)
    _, codes_b, scales_b, ts_b = gpu_quantize(F, d["w"].cuda(), NV, FOS | B2D | TR)
    fwd = oracle.dequantize(NV, codes_f[0], scales_f[0], float(ts_f[0]))
    bwd = oracle.dequantize(NV, codes_b[0], scales_b[0], float(ts_b[0]))
    assert np.array_equal(fwd.T, bwd)


# ---------------------------------------------------------------------------
# full size (the benchmark's 8192^3 launch configuration), sampled outputs
# ---------------------------------------------------------------------------
def sample(n, rng):
    return np.sort(rng.choice(n, size=48, replace=False))


@pytest.fixture(scope="module")
def full_inputs():
    return inputs.training_backward()


def test_full_dgrad(oracle, full_inputs):
    d = full_inputs
    m, n = d["grad"].shape
    k = d["w"].shape[1]
    print(f"[backward-full] dgrad {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(11)
    rows, cols = sample(m, rng), sample(k, rng)
    qg, dg = operand(oracle, d["grad"], FOS | SR, G_OFFSET, rows=rows)
    qwt, dwt = operand(oracle, d["w"], FOS | B2D | TR, rows=cols)
    for out in (torch.bfloat16, torch.float32):
        dx = F.gemm(qg, qwt, out)
        torch.cuda.synchronize()
        check_product(oracle, dx, dg, dwt, out, f"dgrad 8192^3 {out}", rows, cols)
        del dx


def test_full_wgrad(oracle, full_inputs):
    d = full_inputs
    m, n = d["grad"].shape
    k = d["x"].shape[1]
    print(f"[backward-full] wgrad {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(12)
    rows, cols = sample(n, rng), sample(k, rng)
    qgt, dgt = operand(oracle, d["grad"], FOS | SR | TR, GT_OFFSET, rows=rows)
    qxt, dxt = operand(oracle, d["x"], FOS | TR, rows=cols)
    for out in (torch.bfloat16, torch.float32):
        dw = F.gemm(qgt, qxt, out)
        torch.cuda.synchronize()
        check_product(oracle, dw, dgt, dxt, out, f"wgrad 8192^3 {out}", rows, cols)
        del dw
