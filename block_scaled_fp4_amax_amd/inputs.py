"""Seeded synthetic inputs for the five workloads (shapes and distributions
only; none of the quantization method's arithmetic lives here). Shared by the
tests, the smoke check and the benchmark, and by both the GPU path and the
oracle: every generator is deterministic for a given (seed, device).

Workloads (LLM-shaped, synthetic; no dataset or trained weights are used):
  worked_example  4096 fp32 values ~N(0,1), every 512th multiplied by 20
                  (the glossary page's "Como funciona FP4" example).
  w4a4_linear     weight [4096, 4096] ~N(0, 0.02) as [out, in]; activations
                  [2048, 4096] ~N(0, 1) with 1% of the columns (41) x30
                  (outlier channels); bf16.
  moe_mxfp4       32 experts: weight [2880, 5760] ~N(0, 0.02) per expert as
                  [K, N] (quantized transposed); tokens [512, 2880] ~N(0, 1)
                  per expert; bf16.
  training        weight [8192, 8192] ~N(0, 0.02); gradient [8192, 8192]
                  ~Laplace(0, 1e-3) by inverse CDF of a uniform; bf16.
  rht_activation  activations [16384, 4096] ~N(0, 1) with 0.5% of entries
                  replaced by Student-t (df = 2) draws; random 16-bit sign
                  mask; weight [4096, 12288] ~N(0, 0.02) as [K, N]; bf16.
  training_backward  weight [8192, 8192] ~N(0, 0.02), output gradient
                  [8192, 8192] ~Laplace(0, 1e-3), activations [8192, 8192]
                  ~N(0, 1); bf16.
  moe_routed      32 experts as moe_mxfp4, 4096 tokens routed top-4 by
                  logits N(0, 1) plus a per-expert bias 0.5 N(0, 1) (a skewed,
                  load-imbalanced router): per-expert row counts, their
                  offsets, and the routed tokens [sum of counts, 2880]
                  ~N(0, 1) grouped by expert; bf16.
Every size is a parameter so the tests can draw smaller instances from the
same recipe.
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def worked_example(seed: int = 0) -> torch.Tensor:
    g = _gen(seed, "cpu")
    x = torch.randn(4096, generator=g)
    x[::512] *= 20
    return x


def w4a4_linear(m: int = 2048, n: int = 4096, k: int = 4096, seed: int = 2, device="cpu") -> dict:
    g = _gen(seed, device)
    w = (0.02 * torch.randn(n, k, generator=g, device=device)).to(torch.bfloat16)
    a = torch.randn(m, k, generator=g, device=device)
    n_out = max(1, round(0.01 * k))
    cols = torch.randperm(k, generator=g, device=device)[:n_out]
    a[:, cols] *= 30
    return {"w": w, "a": a.to(torch.bfloat16), "outlier_cols": cols}


def moe_mxfp4(experts: int = 32, tokens: int = 512, k: int = 2880, n: int = 5760, seed: int = 3, device="cpu") -> dict:
    g = _gen(seed, device)
    w = torch.empty(experts, k, n, dtype=torch.bfloat16, device=device)
    for e in range(experts):  # per expert, to bound fp32 temporaries
        w[e] = (0.02 * torch.randn(k, n, generator=g, device=device)).to(torch.bfloat16)
    x = torch.randn(experts, tokens, k, generator=g, device=device).to(torch.bfloat16)
    return {"w": w, "x": x}


def training(n: int = 8192, seed: int = 4, device="cpu") -> dict:
    g = _gen(seed, device)
    w = (0.02 * torch.randn(n, n, generator=g, device=device)).to(torch.bfloat16)
    u = torch.rand(n, n, generator=g, device=device) - 0.5
    grad = -1e-3 * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return {"w": w, "grad": grad.to(torch.bfloat16), "sr_seed": seed, "sr_offset": 0}


def training_backward(m: int = 8192, n: int = 8192, k: int = 8192, seed: int = 6, device="cpu") -> dict:
    """Backward pass of a quantized linear Y = X W^T: weight W [n, k]
    0.02 N(0,1), output gradient dY [m, n] Laplace(0, 1e-3) (the training
    gradient's recipe), activations X [m, k] N(0,1); bf16."""
    g = _gen(seed, device)
    w = (0.02 * torch.randn(n, k, generator=g, device=device)).to(torch.bfloat16)
    u = torch.rand(m, n, generator=g, device=device) - 0.5
    grad = -1e-3 * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    x = torch.randn(m, k, generator=g, device=device).to(torch.bfloat16)
    return {"w": w, "grad": grad.to(torch.bfloat16), "x": x, "sr_seed": seed}


def rht_activation(m: int = 16384, k: int = 4096, n: int = 12288, seed: int = 5, device="cpu") -> dict:
    g = _gen(seed, device)
    x = torch.randn(m, k, generator=g, device=device)
    mask = torch.rand(m, k, generator=g, device=device) < 0.005
    z = torch.randn(m, k, generator=g, device=device)
    u = torch.rand(m, k, generator=g, device=device).clamp_min(1e-12)
    t2 = z / torch.sqrt(-torch.log(u))  # Student-t with 2 degrees of freedom
    x = torch.where(mask, t2, x)
    bits = torch.randint(0, 2, (16,), generator=g, device=device).cpu()
    signs = int(sum(int(b) << i for i, b in enumerate(bits.tolist())))
    w = (0.02 * torch.randn(k, n, generator=g, device=device)).to(torch.bfloat16)
    return {"x": x.to(torch.bfloat16), "w": w, "signs": signs}


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor (the oracle's bf16 input form)."""
    return t.contiguous().cpu().view(torch.int16).numpy().view("uint16")


def router_counts(tokens: int, experts: int, topk: int, seed: int, skew: float = 0.5) -> torch.Tensor:
    """Rows per expert from a top-k router over logits N(0, 1) + skew * a
    per-expert bias N(0, 1). int64 [experts]."""
    g = _gen(seed, "cpu")
    bias = skew * torch.randn(experts, generator=g)
    logits = torch.randn(tokens, experts, generator=g) + bias
    top = logits.topk(topk, dim=1).indices
    return torch.bincount(top.flatten(), minlength=experts)


def offsets_of(counts) -> torch.Tensor:
    """Group row offsets (int32, groups + 1 entries) of a list of counts."""
    c = torch.as_tensor(counts, dtype=torch.int64)
    return torch.cat([torch.zeros(1, dtype=torch.int64), c.cumsum(0)]).to(torch.int32)


def moe_routed(experts: int = 32, tokens: int = 4096, topk: int = 4, k: int = 2880, n: int = 5760, seed: int = 7,
               counts=None, device="cpu") -> dict:
    counts = router_counts(tokens, experts, topk, seed) if counts is None else torch.as_tensor(counts)
    offsets = offsets_of(counts)
    g = _gen(seed + 1, device)
    w = torch.empty(experts, k, n, dtype=torch.bfloat16, device=device)
    for e in range(experts):
        w[e] = (0.02 * torch.randn(k, n, generator=g, device=device)).to(torch.bfloat16)
    x = torch.randn(int(offsets[-1]), k, generator=g, device=device).to(torch.bfloat16)
    return {"w": w, "x": x, "counts": counts, "offsets": offsets}
