"""fp4_quantize_noalloc through the C ABI against fp4_quantize (the entry
point with a caller workspace): codes, scale bytes and tensor scales must be
identical, bit for bit, on two calls in a row on the library's shared scratch,
the second with a smaller input, for every kind of pre-pass the scratch
serves (plain, Hadamard rows, Hadamard transposed, batched, the once-folded
large item) and for calls that need no scratch."""
import numpy as np
import pytest
import torch

from gpu_util import flag_str, mixed_matrix

pytestmark = pytest.mark.gpu

MX, NV = 0, 1
FOS, B2D, TR, SR, RHT = 1, 2, 4, 8, 16


def run(F, x, fmt, flags, noalloc, amax=None):
    """One call of either entry point on x [B, rows, cols] bf16 (device);
    returns (codes, scales, tensor scales) as host arrays."""
    B, rows, cols = x.shape
    tr = bool(flags & TR)
    R, C = (cols, rows) if tr else (rows, cols)
    blk = 16 if fmt == NV else 32
    opts = F.make_opts(fmt, flags, 0x3C5A, 99, 7, amax.data_ptr() if amax is not None else 0)
    codes = torch.full((B, R, C // 2), 0xEE, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, R, C // blk), 0xEE, dtype=torch.uint8, device="cuda")
    ts = torch.full((B,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), F.FP4_BF16, B, rows, cols, cols, rows * cols, opts, codes.data_ptr(), C // 2,
            R * (C // 2), scales.data_ptr(), C // blk, R * (C // blk), ts.data_ptr() if fmt == NV else None)
    if noalloc:
        st = F.fp4_quantize_noalloc(*args, stream)
    else:
        wsb = F.fp4_quantize_workspace(B, rows, cols, opts)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
        st = F.fp4_quantize(*args, ws.data_ptr(), wsb, stream)
    assert st == F.FP4_OK, F.fp4_status_str(st)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), ts.cpu().numpy()


CASES = [
    # (fmt, flags, first shape, second (smaller) shape)
    (NV, 0, (1, 640, 1024), (1, 96, 160)),
    (NV, FOS, (3, 256, 512), (2, 64, 96)),
    (NV, FOS | RHT, (1, 512, 768), (1, 48, 64)),
    (NV, FOS | RHT | TR, (2, 512, 256), (1, 64, 64)),
    (NV, B2D | FOS | TR, (1, 512, 512), (1, 64, 128)),
    (NV, FOS | SR, (1, 384, 512), (1, 32, 64)),
    (NV, FOS, (1, 8192, 4096), (1, 1024, 2048)),  # 2^25 elements: the partials are folded once
    (MX, 0, (1, 256, 512), (1, 64, 64)),
]


@pytest.mark.parametrize("fmt,flags,s1,s2", CASES, ids=[f"{f}-{flag_str(g)}-{a}" for f, g, a, _ in CASES])
def test_noalloc_matches_workspace_entry_point(fp4, fmt, flags, s1, s2):
    print(f"[noalloc] fmt={fmt} flags={flag_str(flags)} {s1} then {s2}", flush=True)
    for i, shape in enumerate((s1, s2)):
        x = torch.stack([mixed_matrix(shape[1], shape[2], seed=100 * i + b + flags) * (10.0 ** b)
                         for b in range(shape[0])]).cuda()
        want = run(fp4, x, fmt, flags, noalloc=False)
        got = run(fp4, x, fmt, flags, noalloc=True)
        for w, g, what in zip(want, got, ("codes", "scales", "tensor scale")):
            if what == "tensor scale" and fmt == MX:
                continue
            assert np.array_equal(w.view(np.uint8), g.view(np.uint8)), f"call {i + 1} {shape}: {what} differ"


def test_noalloc_with_caller_amax_needs_no_scratch(fp4):
    x = mixed_matrix(128, 256, seed=5).unsqueeze(0).cuda()
    amax = x.float().abs().amax().reshape(1) * 2
    want = run(fp4, x, NV, FOS, noalloc=False, amax=amax)
    got = run(fp4, x, NV, FOS, noalloc=True, amax=amax)
    for w, g in zip(want, got):
        assert np.array_equal(w.view(np.uint8), g.view(np.uint8))


def test_noalloc_refuses_more_than_its_scratch(fp4):
    """64 items of 8192 x 8192 would need 64 * 4100 bytes of partials: refused
    with FP4_ERR_SCRATCH on the host, before any pointer is touched."""
    opts = fp4.make_opts(NV, 0)
    fake = 0x7F0000000000
    st = fp4.fp4_quantize_noalloc(fake, fp4.FP4_BF16, 64, 8192, 8192, 8192, 8192 * 8192, opts, fake, 4096,
                                  8192 * 4096, fake, 512, 8192 * 512, fake, None)
    assert st == fp4.FP4_ERR_SCRATCH
