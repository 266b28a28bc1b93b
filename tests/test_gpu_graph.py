"""The hot path captured in a HIP graph: NVFP4 4/6 quantize of A and W (each
with its amax pre-pass in the caller's workspace), the GEMM, and the GEMM with
its output quantized in the epilogue, all through the C ABI on the capture
stream. The graph is replayed several times, with new input values written
and other eager work and synchronizations between the replays; every replay
must equal the same calls made eagerly, bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp4_amax_amd as F
from block_scaled_fp4_amax_amd import inputs

pytestmark = pytest.mark.gpu


class Step:
    """Preallocated buffers and the step's C-ABI calls."""

    def __init__(self, M, N, K):
        dev = "cuda"
        self.M, self.N, self.K = M, N, K
        self.xa = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.xw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        self.opts = F.make_opts(F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX)
        self.qa = self._qbuf(M, K)
        self.qw = self._qbuf(N, K)
        self.c = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.amax = torch.tensor([40.0], dtype=torch.float32, device=dev)
        self.out_opts = F.make_opts(F.FP4_NVFP4, F.FP4_FOUR_OVER_SIX, amax_in=self.amax.data_ptr())
        self.qc = self._qbuf(M, N)

    def _qbuf(self, R, C):
        dev = "cuda"
        lds = F.scale_pitch(C // 16)
        ws = F.fp4_quantize_workspace(1, R, C, self.opts)
        return {"codes": torch.empty((R, C // 2), dtype=torch.uint8, device=dev),
                "scales": torch.empty((R, lds), dtype=torch.uint8, device=dev), "lds": lds,
                "ts": torch.empty((1,), dtype=torch.float32, device=dev),
                "ws": torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev), "ws_bytes": ws}

    def _quantize(self, x, q, R, C, stream):
        st = F.fp4_quantize(x.data_ptr(), F.FP4_BF16, 1, R, C, C, R * C, self.opts, q["codes"].data_ptr(), C // 2,
                            R * C // 2, q["scales"].data_ptr(), q["lds"], R * q["lds"], q["ts"].data_ptr(),
                            q["ws"].data_ptr(), q["ws_bytes"], stream)
        assert st == 0, F.fp4_status_str(st)

    def run(self, stream, stream_a=None, stream_w=None):
        M, N, K = self.M, self.N, self.K
        self._quantize(self.xa, self.qa, M, K, stream_a or stream)
        self._quantize(self.xw, self.qw, N, K, stream_w or stream)
        self.gemms(stream)

    def gemms(self, stream):
        M, N, K = self.M, self.N, self.K
        a, w = self.qa, self.qw
        st = F.fp4_gemm(F.FP4_NVFP4, 1, M, N, K, a["codes"].data_ptr(), K // 2, 0, a["scales"].data_ptr(),
                        a["lds"], 0, a["ts"].data_ptr(), w["codes"].data_ptr(), K // 2, 0, w["scales"].data_ptr(),
                        w["lds"], 0, w["ts"].data_ptr(), self.c.data_ptr(), F.FP4_F32, N, 0, stream)
        assert st == 0, F.fp4_status_str(st)
        q = self.qc
        st = F.fp4_gemm_quantize_output(F.FP4_NVFP4, 1, M, N, K, a["codes"].data_ptr(), K // 2, 0,
                                        a["scales"].data_ptr(), a["lds"], 0, a["ts"].data_ptr(),
                                        w["codes"].data_ptr(), K // 2, 0, w["scales"].data_ptr(), w["lds"], 0,
                                        w["ts"].data_ptr(), self.out_opts, q["codes"].data_ptr(), N // 2, 0,
                                        q["scales"].data_ptr(), q["lds"], 0, q["ts"].data_ptr(), stream)
        assert st == 0, F.fp4_status_str(st)

    def outputs(self):
        return [t.clone() for t in (self.qa["codes"], self.qa["scales"], self.qa["ts"], self.qw["codes"],
                                    self.qw["scales"], self.qw["ts"], self.c, self.qc["codes"], self.qc["scales"],
                                    self.qc["ts"])]


def test_graph_replays_match_eager():
    M, N, K = 256, 384, 512
    print(f"[graph] capture quantize x2 + gemm + fused gemm, {M}x{N}x{K}", flush=True)
    step = Step(M, N, K)
    d = inputs.w4a4_linear(m=M, n=N, k=K, seed=1, device="cuda")
    step.xa.copy_(d["a"])
    step.xw.copy_(d["w"])
    step.run(torch.cuda.current_stream().cuda_stream)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(torch.cuda.current_stream().cuda_stream)
    for r in range(4):
        d = inputs.w4a4_linear(m=M, n=N, k=K, seed=10 + r, device="cuda")
        step.xa.copy_(d["a"] * (1.0 + r))
        step.xw.copy_(d["w"])
        _ = (step.c * 2.0).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        step.run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = step.outputs()
        for k, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x, y), f"replay {r}: output {k} differs from the eager call"
        assert float(got[2][0]) != 0.0


def test_graph_with_concurrent_quantizations():
    """The two quantizations captured on two side streams forked from the
    capture stream and joined before the GEMMs (as the benchmark captures its
    steps): every replay equals the eager calls."""
    M, N, K = 320, 256, 384
    print(f"[graph] fork/join capture, {M}x{N}x{K}", flush=True)
    step = Step(M, N, K)
    d = inputs.w4a4_linear(m=M, n=N, k=K, seed=2, device="cuda")
    step.xa.copy_(d["a"])
    step.xw.copy_(d["w"])
    step.run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    sa, sw = torch.cuda.Stream(), torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        main = torch.cuda.current_stream()
        sa.wait_stream(main)
        sw.wait_stream(main)
        step._quantize(step.xa, step.qa, M, K, sa.cuda_stream)
        step._quantize(step.xw, step.qw, N, K, sw.cuda_stream)
        main.wait_stream(sa)
        main.wait_stream(sw)
        step.gemms(main.cuda_stream)
    for r in range(3):
        d = inputs.w4a4_linear(m=M, n=N, k=K, seed=20 + r, device="cuda")
        step.xa.copy_(d["a"])
        step.xw.copy_(d["w"] * (0.5 + r))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        step.run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = step.outputs()
        for k, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x, y), f"replay {r}: output {k} differs from the eager call"
