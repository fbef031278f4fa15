"""Seeded synthetic partial sums for the five workloads and two study inputs.

This module only draws random inputs; it holds none of the method's
arithmetic, and both the GPU path's tests and the CPU oracle's tests take
their inputs from it.  Each rank's partial sums are drawn in float32 and
rounded to bfloat16 (round to nearest even, torch's ``.to(torch.bfloat16)``).

Workloads (shapes from the pages' settings; no dataset or model is used,
the value distributions stand in for the activation and gradient statistics
a tensor-parallel block would produce):

  single    P=4, 64 tokens x hidden 1024; N(0,1) with 0.1 % of the elements
            (66 per rank, chosen by randperm) multiplied by 20.
  chain     P=4, 2048 x 4096, 64 sites; 0.02 * N(0,1) * sigma_h, where the
            per-channel scale sigma_h = exp(N(0,1)) (lognormal, sigma = 1) is
            drawn once per chain and shared by ranks and sites.
  onegb     P=4 or 8, 2^29 elements (1 GiB of bf16) per rank, Laplace(0,1);
            drawn on the GPU with torch's device generator.
  chain8    P=4, 4096 x 1024, 56 sites, 8-bit; N(0, 0.05) where a
            Bernoulli(0.3) mask replaces values by U(-1e-3, 1e-3).
  training  P=4, 32 x 4096 x 1024 per rank, 28 layers x 2 sites, forward then
            backward; forward N(0,1); backward N(0, 1e-3) with 0.05 % of the
            elements multiplied by 50.
  tpblock   the operands of one rank's row-parallel matmul, A [M, K] and
            W [N, K] in bf16: "normal" draws activations N(0,1) and weights
            N(0, 1/K) (random init, so the partial sums have unit scale);
            "int" draws small integers (A in [-4, 4], W in [-3, 3]), whose
            products and sums are exact in fp32 at any summation order;
            "ternary" draws A and W in {-1, 0, 1} (as int8, so that operands
            of billions of elements fit), whose partial sums stay exact in
            fp32 for any K below 2^24.
            Default shape: a Llama-3-8B MLP down projection at TP = 4 (4096
            tokens, hidden 4096, K = 14336 / 4 = 3584).
  sparse    the chain workload's values with a Bernoulli(keep) mask of exact
            zeros (keep = 0.5 by default): partial sums of sparse activations,
            where most groups hold both signs and many exact zeros.
  shifted   the chain workload's values plus a per-channel positive mean
            0.15 * |N(0,1)| * sigma_h (drawn once), so that many groups are
            one-sided, as after a gated or rectified activation.

Seed of (workload, step, site, rank): 20261202 + 1000003*w + 10007*step +
101*site + rank, with w = 1..8 in the order above.
"""
from __future__ import annotations

import math

import torch

WORKLOADS = {"single": 1, "chain": 2, "onegb": 3, "chain8": 4, "training": 5, "tpblock": 6, "sparse": 7,
             "shifted": 8}

SHAPES = {
    "single": dict(P=4, tokens=64, hidden=1024, bits=4, sites=1),
    "chain": dict(P=4, tokens=2048, hidden=4096, bits=4, sites=64),
    "onegb": dict(P=4, tokens=1, hidden=1 << 29, bits=4, sites=1),
    "chain8": dict(P=4, tokens=4096, hidden=1024, bits=8, sites=56),
    "training": dict(P=4, tokens=32 * 4096, hidden=1024, bits=4, sites=56),
    "tpblock": dict(P=4, tokens=4096, hidden=4096, bits=4, sites=1, k=14336 // 4),
}


def seed_of(workload: str, step: int = 0, site: int = 0, rank: int = 0) -> int:
    return 20261202 + 1000003 * WORKLOADS[workload] + 10007 * step + 101 * site + rank


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _bf16_bits(x32: torch.Tensor) -> torch.Tensor:
    """float32 -> bfloat16 (nearest even) -> int16 view of the bit patterns."""
    return x32.to(torch.bfloat16).view(torch.int16)


def single(rank: int, n: int = 64 * 1024, seed_step: int = 0) -> torch.Tensor:
    g = _gen(seed_of("single", seed_step, 0, rank))
    x = torch.randn(n, generator=g, dtype=torch.float32)
    k = int(math.ceil(0.001 * n))
    idx = torch.randperm(n, generator=g)[:k]
    x[idx] *= 20.0
    return _bf16_bits(x)


def chain_channel_scale(hidden: int = 4096, chain_seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed_of("chain", 0, 0, 0) + 7 + chain_seed, device=device)
    return torch.exp(torch.randn(hidden, generator=g, dtype=torch.float32, device=device))


def chain(rank: int, site: int, tokens: int = 2048, hidden: int = 4096,
          sigma_h: torch.Tensor | None = None, chain_seed: int = 0, device="cpu") -> torch.Tensor:
    if sigma_h is None:
        sigma_h = chain_channel_scale(hidden, chain_seed, device=device)
    g = _gen(seed_of("chain", chain_seed, site, rank), device=device)
    x = 0.02 * torch.randn(tokens, hidden, generator=g, dtype=torch.float32, device=device) * sigma_h
    return _bf16_bits(x.reshape(-1))


def sparse(rank: int, site: int, tokens: int, hidden: int, sigma_h: torch.Tensor, keep: float = 0.5,
           device="cpu") -> torch.Tensor:
    g = _gen(seed_of("sparse", 0, site, rank), device=device)
    x = 0.02 * torch.randn(tokens, hidden, generator=g, dtype=torch.float32, device=device) * sigma_h
    mask = torch.rand(tokens, hidden, generator=g, device=device) < keep
    x = torch.where(mask, x, torch.zeros((), device=device))
    return _bf16_bits(x.reshape(-1))


def shifted(rank: int, site: int, tokens: int, hidden: int, sigma_h: torch.Tensor, device="cpu") -> torch.Tensor:
    gm = _gen(seed_of("shifted", 0, 0, 0) + 7, device=device)
    mu = 0.15 * torch.randn(hidden, generator=gm, dtype=torch.float32, device=device).abs() * sigma_h
    g = _gen(seed_of("shifted", 0, site, rank), device=device)
    x = 0.02 * torch.randn(tokens, hidden, generator=g, dtype=torch.float32, device=device) * sigma_h + mu
    return _bf16_bits(x.reshape(-1))


def chain8(rank: int, site: int, tokens: int = 4096, hidden: int = 1024,
           chain_seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed_of("chain8", chain_seed, site, rank), device=device)
    n = tokens * hidden
    x = 0.05 * torch.randn(n, generator=g, dtype=torch.float32, device=device)
    mask = torch.rand(n, generator=g, device=device) < 0.3
    small = (torch.rand(n, generator=g, dtype=torch.float32, device=device) * 2.0 - 1.0) * 1e-3
    x = torch.where(mask, small, x)
    return _bf16_bits(x)


def training(rank: int, step: int, site: int, backward: bool, n: int,
             device="cpu") -> torch.Tensor:
    """One site's partial sums; site numbers 0..55 forward, 56..111 backward."""
    g = _gen(seed_of("training", step, site, rank), device=device)
    if not backward:
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device)
    else:
        x = 1e-3 * torch.randn(n, generator=g, dtype=torch.float32, device=device)
        k = int(math.ceil(0.0005 * n))
        idx = torch.randint(0, n, (k,), generator=g, device=device)
        x[idx] *= 50.0
    return _bf16_bits(x)


def laplace(rank: int, n: int, device="cpu", chunk: int = 1 << 26, workload: str = "onegb") -> torch.Tensor:
    """Laplace(0, 1) by inversion of a uniform draw, generated in chunks so
    that the float32 temporaries stay small next to a 1 GiB output.  |u - 1/2|
    is kept below 1/2 (a draw of exactly 0 would give log(0) = -inf), which caps
    |x| at 24*ln 2 = 16.6."""
    g = _gen(seed_of(workload, 0, 0, rank), device=device)
    out = torch.empty(n, dtype=torch.int16, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        u = torch.rand(b - a, generator=g, dtype=torch.float32, device=device)
        out[a:b] = _bf16_bits(laplace_from_uniform(u))
        del u
    return out


# the largest float32 below 1/2 (0.5 - 2^-26 would round back to 0.5)
_HALF_BELOW = 0.5 - 2.0 ** -25


def laplace_from_uniform(u: torch.Tensor) -> torch.Tensor:
    """Laplace(0, 1) from U[0, 1) draws by inversion, finite for every draw."""
    c = u - 0.5
    return -torch.sign(c) * torch.log1p(-2.0 * c.abs().clamp(max=_HALF_BELOW))


def tp_operands(rank: int, M: int, N: int, K: int, kind: str = "normal", site: int = 0, device="cpu"):
    """A [M, K] and W [N, K] (bf16 bit tensors, int16) of one rank's
    row-parallel matmul; see the module docstring."""
    g = _gen(seed_of("tpblock", 0, site, rank), device=device)
    if kind == "int":
        a = torch.randint(-4, 5, (M, K), generator=g, device=device).to(torch.float32)
        w = torch.randint(-3, 4, (N, K), generator=g, device=device).to(torch.float32)
    elif kind == "ternary":
        a = torch.randint(-1, 2, (M, K), generator=g, device=device, dtype=torch.int8)
        w = torch.randint(-1, 2, (N, K), generator=g, device=device, dtype=torch.int8)
        return a.to(torch.bfloat16).view(torch.int16), w.to(torch.bfloat16).view(torch.int16)
    elif kind == "normal":
        a = torch.randn(M, K, generator=g, dtype=torch.float32, device=device)
        w = torch.randn(N, K, generator=g, dtype=torch.float32, device=device) * (1.0 / math.sqrt(K))
    else:
        raise ValueError(kind)
    return _bf16_bits(a), _bf16_bits(w)


def as_numpy_u16(t: torch.Tensor):
    """Host copy of a bf16-bit tensor as a numpy uint16 array."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
