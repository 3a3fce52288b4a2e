"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and names workloads; it holds none of the
method's arithmetic, so the oracle and the HIP path can both take their inputs
from it without sharing any computation.

Recipe (the shapes are the workloads the library is measured on):
  * every tensor is [B, H, N, d] row-major (decode vectors are [B, H, d]);
  * Q, K, V ~ N(0, 1), scaled by 1/sqrt(d) when ``scale`` is set, drawn in
    fp32 and rounded to the target dtype (round-to-nearest-even for bf16);
  * the output gradient dO ~ N(0, 1) in the target dtype;
  * FAVOR+ random directions (``favor_omega``): a [d, d] fp32 matrix with rows
    ~ N(0, I_d), from its own seeded generator (i.i.d., or orthogonal within each
    block of d rows); FAVOR+ queries and keys
    (``favor_qkv``) ~ N(0, 1) d^(-1/4), the page's pre-normalization;
  * draws come from one torch.Generator seeded with ``seed``, in the order
    q, k, v, dout.  ``device="cuda"`` draws with the device generator (fast for
    the multi-GiB workloads); tests copy the exact drawn values to the host.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    scale: bool          # divide Q, K, V by sqrt(d)
    chunk: int = 64
    calls: tuple = ()


# The five measured workloads.
TINY = Workload("tiny", 1, 2, 256, 32, torch.float32, False,
                calls=("fwd_noncausal", "fwd_causal", "bwd_causal"))
MID = Workload("mid", 4, 16, 4096, 64, torch.bfloat16, True,
               calls=("fwd_causal", "bwd_causal", "fwd_noncausal"))
LONG = Workload("long", 8, 16, 16384, 128, torch.bfloat16, True, calls=("fwd_causal", "bwd_causal"))
VERYLONG = Workload("verylong", 1, 32, 131072, 128, torch.bfloat16, True, calls=("fwd_causal",))


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    H: int
    d: int
    prefix: int
    steps: int
    dtype: torch.dtype


DECODE = DecodeWorkload("decode", 256, 32, 128, 2048, 512, torch.bfloat16)

WORKLOADS = {w.name: w for w in (TINY, MID, LONG, VERYLONG)}


def generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, gen: torch.Generator, dtype: torch.dtype, scale: float = 1.0,
           device: str = "cpu") -> torch.Tensor:
    """N(0, 1) * scale drawn in fp32, then rounded to ``dtype``."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def qkv(B, H, N, d, dtype=torch.bfloat16, seed=0, scale=True, device="cpu", with_dout=False):
    """Draw q, k, v (and dout) of shape [B, H, N, d] in that order from one generator."""
    gen = generator(seed, device)
    s = 1.0 / math.sqrt(d) if scale else 1.0
    q = normal((B, H, N, d), gen, dtype, s, device)
    k = normal((B, H, N, d), gen, dtype, s, device)
    v = normal((B, H, N, d), gen, dtype, s, device)
    if not with_dout:
        return q, k, v
    dout = normal((B, H, N, d), gen, dtype, 1.0, device)
    return q, k, v, dout


def workload_inputs(w: Workload, seed=0, device="cpu", with_dout=True):
    return qkv(w.B, w.H, w.N, w.d, w.dtype, seed, w.scale, device, with_dout)


def decode_tokens(batch, H, d, steps, dtype=torch.bfloat16, seed=1, device="cpu"):
    """Per-step decode vectors q, k, v of shape [steps, batch, H, d] ~ N(0,1)/sqrt(d)."""
    gen = generator(seed, device)
    s = 1.0 / math.sqrt(d)
    q = normal((steps, batch, H, d), gen, dtype, s, device)
    k = normal((steps, batch, H, d), gen, dtype, s, device)
    v = normal((steps, batch, H, d), gen, dtype, s, device)
    return q, k, v


def favor_qkv(B, H, N, d, dtype=torch.bfloat16, seed=0, device="cpu", with_dout=False):
    """Inputs of the FAVOR+ path: q, k ~ N(0, 1) d^(-1/4) (the pre-normalization that puts
    the softmax's 1/sqrt(d) into q.k), v ~ N(0, 1)/sqrt(d), dout ~ N(0, 1); same draw order."""
    gen = generator(seed, device)
    sqk = d ** -0.25
    q = normal((B, H, N, d), gen, dtype, sqk, device)
    k = normal((B, H, N, d), gen, dtype, sqk, device)
    v = normal((B, H, N, d), gen, dtype, 1.0 / math.sqrt(d), device)
    if not with_dout:
        return q, k, v
    return q, k, v, normal((B, H, N, d), gen, dtype, 1.0, device)


def favor_omega(d, seed=0, device="cpu", m=None, orthogonal=False):
    """FAVOR+ random directions: an [m, d] fp32 matrix (m = d by default) whose rows are drawn from N(0, I_d).

    orthogonal: within every block of d rows the directions are exactly orthogonal (the Performer
    section's orthogonal random features, which lower the estimate's variance below i.i.d. draws):
    each block is the orthogonal factor of a QR decomposition of a d x d Gaussian matrix (column
    signs fixed by R's diagonal, so the factor is Haar distributed), its rows scaled by the norms
    of independent N(0, I_d) vectors, so that every row on its own is still distributed N(0, I_d)."""
    m = d if m is None else m
    gen = generator(seed, device)
    if not orthogonal:
        return torch.randn((m, d), generator=gen, dtype=torch.float32, device=device)
    blocks = []
    for _ in range((m + d - 1) // d):
        g = torch.randn((d, d), generator=gen, dtype=torch.float64, device=device)
        qf, r = torch.linalg.qr(g)
        qf = qf * torch.sign(torch.diagonal(r))[None, :]
        norms = torch.randn((d, d), generator=gen, dtype=torch.float64, device=device).norm(dim=1)
        blocks.append(qf.T * norms[:, None])
    return torch.cat(blocks)[:m].to(torch.float32)


def to_f64(x: torch.Tensor):
    """Exact widening of a tensor's values to a float64 numpy array on the host."""
    return x.detach().to("cpu", torch.float64).numpy()
