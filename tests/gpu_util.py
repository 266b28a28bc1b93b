"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same inputs."""
import numpy as np
import torch

from block_scaled_fp4_amax_amd import inputs

FLAG_NAMES = {1: "fos", 2: "b2d", 4: "tr", 8: "sr", 16: "rht", 32: "search", 64: "tensor"}


def flag_str(flags):
    return "+".join(n for b, n in FLAG_NAMES.items() if flags & b) or "plain"


def oracle_input(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return inputs.bf16_bits(t)
    return t.float().numpy()


def oracle_quantize(O, x: torch.Tensor, fmt, flags=0, signs=0, seed=0, offset=0, amax=None):
    """x: [B, rows, cols] (or 2-D) CPU tensor. Oracle codes/scales/tensor scale
    per batch item, with the stochastic-rounding index running over the whole
    batched output."""
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    B, rows, cols = x3.shape
    R, C = (cols, rows) if flags & O.TRANSPOSE else (rows, cols)
    codes, scales, ts = [], [], []
    for b in range(B):
        a = None if amax is None else float(amax[b])
        r = O.quantize(oracle_input(x3[b]), fmt, flags=flags, rht_signs=signs, seed=seed, offset=offset, amax=a,
                       L0=b * R * C)
        codes.append(r["codes"])
        scales.append(r["scales"])
        ts.append(r["tensor_scale"] if r["tensor_scale"] is not None else 0.0)
    return np.stack(codes), np.stack(scales), np.array(ts, np.float32)


def gpu_quantize(F, x_dev: torch.Tensor, fmt, flags=0, signs=0, seed=0, offset=0, amax=None):
    q = F.quantize(x_dev, fmt, four_over_six=bool(flags & 1), block2d=bool(flags & 2), transpose=bool(flags & 4),
                   stochastic=bool(flags & 8), hadamard=bool(flags & 16), scale_search=bool(flags & 32),
                   tensor_scale=bool(flags & 64), rht_signs=signs, seed=seed, offset=offset, amax=amax)
    torch.cuda.synchronize()
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    ts = q.tensor_scale.cpu().numpy() if q.tensor_scale is not None else None
    if codes.ndim == 2:
        codes, scales = codes[None], scales[None]
    return q, codes, scales, ts


def assert_codes_equal(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} bytes differ; first at {i}: "
                             f"gpu=0x{int(got[i]):02x} oracle=0x{int(want[i]):02x}")


def mixed_matrix(rows, cols, seed, dtype=torch.bfloat16, device="cpu"):
    """Normal values with per-row magnitude spread, outliers, a zero row, a
    row of tiny values and exact E2M1 midpoints (rounding ties)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * torch.exp(torch.empty(rows, 1).uniform_(-4, 4, generator=g))
    x[torch.rand(rows, cols, generator=g) < 0.01] *= 40
    if rows > 3:
        x[1] = 0.0
        x[2] = x[2] * 1e-30
        x[3, : min(cols, 32)] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)[: min(cols, 32)]
        x[3, 0] = 6.0
    return x.to(dtype).to(device)


def upload_scales(scales):
    """Upload a [.., R, nb] uint8 scale array with rows padded to the 16-byte
    pitch fp4_gemm reads; returns the [.., R, nb] view."""
    import block_scaled_fp4_amax_amd as F
    a = np.asarray(scales, dtype=np.uint8)
    nb = a.shape[-1]
    buf = np.zeros((*a.shape[:-1], F.scale_pitch(nb)), dtype=np.uint8)
    buf[..., :nb] = a
    return torch.from_numpy(buf).cuda()[..., :nb]


def check_close(c_gpu, ref, absab, K, out_dtype, what):
    c = c_gpu.double().cpu().numpy()
    bound = (2 * K + 4) * 2.0 ** -24 * absab
    if out_dtype == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(c - ref)
    worst = np.argmax(err - bound)
    assert (err <= bound + 1e-30).all(), f"{what}: element bound exceeded at {np.unravel_index(worst, err.shape)}"
    if out_dtype == torch.float32:
        rel = np.linalg.norm(c - ref) / max(np.linalg.norm(ref), 1e-300)
        assert rel <= 1e-3, f"{what}: relative Frobenius error {rel}"


def oracle_operand(O, x, fmt, flags, signs=0, rows=None):
    """Oracle-quantize x ([G, r, c] CPU). Returns the uploaded Quantized and the
    oracle's dequantized values [G, R, C] (float32), optionally only for the
    output rows `rows`."""
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    codes, scales, ts, deq = [], [], [], []
    for b in range(x3.shape[0]):
        r = O.quantize(oracle_input(x3[b]), fmt, flags=flags, rht_signs=signs)
        codes.append(r["codes"])
        scales.append(r["scales"])
        ts.append(r["tensor_scale"] or 0.0)
        c, s = (r["codes"], r["scales"]) if rows is None else (r["codes"][rows], r["scales"][rows])
        deq.append(O.dequantize(fmt, c, s, r["tensor_scale"]))
    import block_scaled_fp4_amax_amd as F
    q = F.Quantized(fmt, torch.from_numpy(np.stack(codes)).cuda(), upload_scales(np.stack(scales)),
                    torch.tensor(ts, dtype=torch.float32).cuda() if fmt == O.NVFP4 else None)
    return q, np.stack(deq)
