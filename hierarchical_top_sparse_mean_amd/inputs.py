"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the attention method itself: it only draws
the tensors that both the HIP path and the CPU oracle consume.

Recipe (every workload):
  1. ``g = torch.Generator('cpu').manual_seed(seed)`` (seed 0 by default);
  2. draw Q, K, V and then dO, in that order, each
     ``torch.randn([batch, heads, N, d], generator=g, dtype=torch.float32)``;
  3. structured workloads add one shared smooth 2D sinusoid to Q, K and V
     (same for every batch and head).  The tokens are the pixels of an S x S
     image in raster order (S = sqrt(N)); token t sits at y = t // S,
     x = t % S; channel c uses the spatial frequency
     (fx, fy) = [(0, 1), (1, 0), (1, 1), (1, -1)][c % 4] and phase
     2*pi*c/d:  s[t, c] = sin(2*pi*(fx*x + fy*y)/S + 2*pi*c/d), amplitude 1,
     evaluated in float64 and rounded to float32;
  4. cast to the workload's dtype (bfloat16 by round-to-nearest-even).

The image workloads of the method's evaluation (pixel-space generation at
32x32 ... 512x512) are stood in for by these synthetic tokens of the same
sequence lengths; no dataset is read.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    dtype: torch.dtype
    block: int
    levels: int          # pooling steps: seq_len -> seq_len/B -> ... -> seq_len/B^levels
    topk: int
    enrich: int          # coarse levels 2..enrich+1 enrich the attended set
    backward: bool
    sinusoid: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def bh(self) -> int:
        return self.batch * self.heads

    def describe(self) -> str:
        chain = "->".join(str(self.seq_len // self.block ** l) for l in range(self.levels + 1))
        return (f"{self.name}: {self.batch}x{self.heads}x{self.seq_len} d={self.head_dim} "
                f"{str(self.dtype).replace('torch.', '')} B={self.block} chain {chain} "
                f"K={self.topk} Le={self.enrich} {'fwd+bwd' if self.backward else 'fwd'}")


WORKLOADS = {
    # 32x32 pixel tokens, iid N(0,1), fp32
    "tiny_n1024_fp32": Workload("tiny_n1024_fp32", 1, 2, 1024, 64, torch.float32, 16, 2, 2, 1,
                                True, False),
    # 64x64 pixel tokens + sinusoid, forward only
    "n4096_bf16": Workload("n4096_bf16", 4, 8, 4096, 64, torch.bfloat16, 16, 2, 8, 1,
                           False, True),
    # 128x128 pixel tokens + sinusoid, forward + backward
    "n16384_bf16": Workload("n16384_bf16", 2, 16, 16384, 64, torch.bfloat16, 16, 2, 8, 1,
                            True, True),
    # 256x256 pixel tokens + sinusoid, forward + backward (the measured workload)
    "n65536_bf16": Workload("n65536_bf16", 1, 16, 65536, 64, torch.bfloat16, 16, 2, 8, 1,
                            True, True),
    # 512x512 pixel tokens + sinusoid, three pooling steps, forward only
    "n262144_bf16": Workload("n262144_bf16", 1, 8, 262144, 64, torch.bfloat16, 16, 3, 8, 2,
                             False, True),
}


def sinusoid(N: int, d: int) -> torch.Tensor:
    """Shared smooth 2D pattern s[t, c] (float32, [N, d]); see the module docstring."""
    S = int(round(math.sqrt(N)))
    if S * S != N:
        raise ValueError("sinusoid needs a square token grid")
    t = torch.arange(N, dtype=torch.float64)
    y = torch.div(t, S, rounding_mode="floor")
    x = t - y * S
    freqs = [(0.0, 1.0), (1.0, 0.0), (1.0, 1.0), (1.0, -1.0)]
    cols = []
    for c in range(d):
        fx, fy = freqs[c % 4]
        cols.append(torch.sin(2.0 * math.pi * (fx * x + fy * y) / S + 2.0 * math.pi * c / d))
    return torch.stack(cols, dim=1).to(torch.float32)


def make_inputs(batch: int, heads: int, N: int, d: int, dtype: torch.dtype,
                sinus: bool, with_grad: bool, seed: int = 0):
    """Returns (q, k, v, dout or None) as CPU tensors of shape [batch, heads, N, d]."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = [batch, heads, N, d]
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    dout = torch.randn(shape, generator=g, dtype=torch.float32) if with_grad else None
    if sinus:
        s = sinusoid(N, d)
        q += s
        k += s
        v += s
    cast = (lambda a: a.to(dtype)) if dtype != torch.float32 else (lambda a: a)
    q, k, v = cast(q), cast(k), cast(v)
    if dout is not None:
        dout = cast(dout)
    return q, k, v, dout


def workload_inputs(w: Workload, seed: int = 0):
    return make_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.sinusoid,
                       w.backward, seed)
