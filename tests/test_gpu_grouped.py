"""GPU parity of fp4_gemm_grouped, the mixture-of-experts grouped GEMM whose
per-group row counts come from a router and live in device memory, against
the oracle's grouped reference (dequantize, then a float64 matmul per
group's row range). Operands are the oracle's codes and scales, uploaded.
Bounds are those of the plain GEMM, per output element."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as F
from block_scaled_fp4_amax_amd import inputs
from gpu_util import check_close, oracle_operand

pytestmark = pytest.mark.gpu

MX, NV = 0, 1
FOS, TR = 1, 4

# group row counts: empty groups, single rows, exact and ragged multiples of
# the 256-row tile, a group spanning several tiles
COUNTS = {
    "mixed": [0, 1, 256, 37, 0, 300, 513, 2],
    "all-empty-but-one": [0, 0, 70, 0],
    "one-group": [200],
    "tile-edges": [255, 257, 256, 511],
}


def operands(O, fmt, counts, k, n, seed):
    d = inputs.moe_routed(experts=len(counts), k=k, n=n, seed=seed, counts=counts)
    fl = FOS if fmt == NV else 0
    qa, da = oracle_operand(O, d["x"], fmt, fl)
    qb, db = oracle_operand(O, d["w"], fmt, fl | TR)
    a = F.Quantized(fmt, qa.codes[0], qa.scales[0], qa.tensor_scale)
    return a, qb, da[0], db, d["offsets"]


def check_groups(O, c, da, db, offsets, out, what, rows=None, cols=None):
    """c [M, N] from the GPU; da [M, K]; db [G, n, K], already restricted to
    the output columns `cols` when those are given; rows: output rows to
    check (default all)."""
    ref = O.grouped_gemm_reference(da, db, offsets.tolist())
    rows = np.arange(c.shape[0]) if rows is None else rows
    if cols is not None:
        c = c[:, torch.from_numpy(cols).cuda()]
    c = c[torch.from_numpy(rows).cuda()]
    ref = ref[rows]
    off = offsets.numpy()
    for g in range(db.shape[0]):
        sel = np.nonzero((rows >= off[g]) & (rows < off[g + 1]))[0]
        if len(sel) == 0:
            continue
        absab = np.abs(da[rows[sel]]).astype(np.float64) @ np.abs(db[g]).astype(np.float64).T
        check_close(c[torch.from_numpy(sel).cuda()], ref[sel], absab, da.shape[-1], out, f"{what} group {g}")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("fmt", [MX, NV], ids=["mx", "nv"])
@pytest.mark.parametrize("case", list(COUNTS))
def test_grouped_counts(oracle, case, fmt, out):
    counts = COUNTS[case]
    print(f"[grouped] {case} counts={counts} fmt={fmt} -> {out}", flush=True)
    a, b, da, db, offsets = operands(oracle, fmt, counts, 192, 136, seed=len(counts))
    c = F.gemm_grouped(a, b, offsets.cuda(), out)
    torch.cuda.synchronize()
    check_groups(oracle, c, da, db, offsets, out, case)


@pytest.mark.parametrize("fmt", [MX, NV], ids=["mx", "nv"])
def test_rows_outside_groups_untouched(oracle, fmt):
    """Rows before the first offset and after the last are not written; an
    offset past M is clamped to M."""
    print(f"[grouped] rows outside groups fmt={fmt}", flush=True)
    counts = [40, 90, 0, 130]
    a, b, da, db, offsets = operands(oracle, fmt, counts, 128, 72, seed=9)
    M, N = da.shape[0], db.shape[1]
    off = torch.tensor([5, 40, 130, 130, M + 100], dtype=torch.int32)
    c = torch.full((M, N), 12345.0, dtype=torch.float32, device="cuda")
    half = a.codes.shape[1]
    st = F.fp4_gemm_grouped(fmt, 4, off.cuda().data_ptr(), M, N, 2 * half, a.codes.data_ptr(), half,
                            a.scales.data_ptr(), a.scales.stride(0),
                            a.tensor_scale.data_ptr() if a.tensor_scale is not None else None,
                            b.codes.data_ptr(), half, N * half, b.scales.data_ptr(), b.scales.stride(1),
                            b.scales.stride(0), b.tensor_scale.data_ptr() if b.tensor_scale is not None else None,
                            c.data_ptr(), F.FP4_F32, N, torch.cuda.current_stream().cuda_stream)
    assert st == 0, F.fp4_status_str(st)
    torch.cuda.synchronize()
    assert (c[:5] == 12345.0).all()
    clamped = torch.tensor([5, 40, 130, 130, M], dtype=torch.int32)
    check_groups(oracle, c, da, db, clamped, torch.float32, "clamped")


def test_router_offsets_computed_on_device(oracle):
    """The offsets can be produced on the device (a cumulative sum of a
    router's counts) and used without a host round trip."""
    counts = [64, 0, 200, 33]
    a, b, da, db, offsets = operands(oracle, MX, counts, 128, 64, seed=4)
    dev_counts = torch.tensor(counts, device="cuda")
    dev_off = torch.cat([torch.zeros(1, dtype=torch.int64, device="cuda"), dev_counts.cumsum(0)]).to(torch.int32)
    c = F.gemm_grouped(a, b, dev_off, torch.float32)
    torch.cuda.synchronize()
    check_groups(oracle, c, da, db, offsets, torch.float32, "device offsets")


def test_full_moe_routed(oracle):
    """The benchmark's shape: 32 experts, 4096 tokens routed top-4 (16384
    rows), K 2880, N 5760, MXFP4, bf16 and fp32 out; sampled rows and
    columns."""
    d = inputs.moe_routed()
    print(f"[grouped-full] counts={d['counts'].tolist()}", flush=True)
    rng = np.random.default_rng(3)
    M, N = d["x"].shape[0], d["w"].shape[2]
    rows = np.sort(rng.choice(M, size=64, replace=False))
    cols = np.sort(rng.choice(N, size=48, replace=False))
    qa, da = oracle_operand(oracle, d["x"], MX, 0)
    qb, db = oracle_operand(oracle, d["w"], MX, TR, rows=cols)
    a = F.Quantized(MX, qa.codes[0], qa.scales[0], None)
    da = da[0]
    for out in (torch.bfloat16, torch.float32):
        c = F.gemm_grouped(a, qb, d["offsets"].cuda(), out)
        torch.cuda.synchronize()
        check_groups(oracle, c, da, db, d["offsets"], out, f"moe routed {out}", rows=rows, cols=cols)
