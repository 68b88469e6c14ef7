"""Seeded synthetic inputs for the Float8Linear workloads.

This module only draws random bf16 tensors; it holds none of the method's
arithmetic, and both the HIP path's tests/benchmark and the oracle's checks
take their inputs from it.

Recipe (one torch CPU generator per workload, seeded; draws in float32, then
rounded to bf16 with torch's round-to-nearest-even):
  * X  ~ N(0, 1)          shape (M, K)
  * W  ~ N(0, 1/fan_in)   shape (N, K), fan_in = K  (std = 1/sqrt(K))
  * dY ~ N(0, 1e-3)       shape (M, N)              (std = sqrt(1e-3))
  N(0, v) names the variance.  Draw order per linear: X, [outlier mask], W, dY.
  Outliers: after X is drawn, mask = rand(M, K) < fraction from the same
  generator, and X[mask] *= multiplier (in float32, before the bf16 rounding).

Workload shapes follow the pages:
  * single linear (4096 -> 4096) at input rows 16, 256, 4096, 65536
    (pytorch/torchtitan PR #778, single-linear-layer table);
  * a Llama-3-8B layer at batch 1 x seq 8192 (PR #778, training table:
    Llama3 8b, batch size 1, seq len 8192; linear shapes from the model's
    dims: d_model 4096, 8 KV heads of 128, FFN 14336);
  * a GPT-1.5B block at batch 12 x seq 1024 (pytorch/ao issue #1297, repro
    script: d_embd 1600, attn_proj 3*d, out_proj d, FFN 4*d), delayed
    scaling, a fresh seed per step.
A workload may name groups of linears that read one input (the q, k, v
projections, the gated MLP's w1 and w3): only the group's first linear
draws X; the others reuse it and draw only W and dY.
"""
from dataclasses import dataclass
from typing import List, Tuple

import torch

X_STD = 1.0
DY_STD = 1e-3 ** 0.5


@dataclass(frozen=True)
class Linear:
    name: str
    M: int  # tokens (rows of X and dY)
    K: int  # in_features
    N: int  # out_features

    @property
    def flops(self) -> int:
        """Forward + backward flops: three GEMMs of 2*M*N*K each."""
        return 6 * self.M * self.N * self.K


@dataclass(frozen=True)
class Workload:
    name: str
    linears: Tuple[Linear, ...]
    scaling: str = "dynamic"  # or "delayed"
    steps: int = 1
    outlier_fraction: float = 0.0
    outlier_multiplier: float = 200.0
    seed: int = 0
    description: str = ""
    shared_x: Tuple[Tuple[str, ...], ...] = ()  # groups of linears reading the same X

    @property
    def flops(self) -> int:
        return sum(l.flops for l in self.linears)


def _llama_layer(m):
    return (Linear("q", m, 4096, 4096), Linear("k", m, 4096, 1024), Linear("v", m, 4096, 1024),
            Linear("o", m, 4096, 4096), Linear("w1", m, 4096, 14336), Linear("w3", m, 4096, 14336),
            Linear("w2", m, 14336, 4096))


def _gpt_block(m):
    return (Linear("qkv", m, 1600, 4800), Linear("out", m, 1600, 1600), Linear("fc1", m, 1600, 6400),
            Linear("fc2", m, 6400, 1600))


WORKLOADS = {
    "linear4096_m16": Workload("linear4096_m16", (Linear("linear", 16, 4096, 4096),),
                               description="single 4096->4096 linear, 16 input rows, dynamic"),
    "linear4096_m256": Workload("linear4096_m256", (Linear("linear", 256, 4096, 4096),),
                                description="single 4096->4096 linear, 256 input rows, dynamic"),
    "linear4096_m4096": Workload("linear4096_m4096", (Linear("linear", 4096, 4096, 4096),),
                                 description="single 4096->4096 linear, 4096 input rows, dynamic"),
    "linear4096_m65536_outliers": Workload(
        "linear4096_m65536_outliers", (Linear("linear", 65536, 4096, 4096),), outlier_fraction=1e-3,
        description="single 4096->4096 linear, 65536 input rows, 0.1% of X scaled x200, dynamic"),
    "llama3_8b_layer_t8192": Workload("llama3_8b_layer_t8192", _llama_layer(8192),
                                      description="Llama-3-8B layer linears (q,k,v,o,w1,w3,w2), 8192 tokens"),
    "llama3_8b_layer_t8192_shared": Workload(
        "llama3_8b_layer_t8192_shared", _llama_layer(8192), shared_x=(("q", "k", "v"), ("w1", "w3")),
        description="Llama-3-8B layer linears, 8192 tokens; q,k,v and w1,w3 read one input each (cast once)"),
    "gpt1p5b_block_t12288_delayed": Workload(
        "gpt1p5b_block_t12288_delayed", _gpt_block(12288), scaling="delayed", steps=20,
        description="GPT-1.5B block linears (qkv,out,fc1,fc2), 12288 tokens, delayed scaling, 20 steps"),
}


def draw_linear(gen: torch.Generator, lin: Linear, outlier_fraction: float = 0.0,
                outlier_multiplier: float = 200.0, x: torch.Tensor = None):
    """Draws (X, W, dY) as bf16 CPU tensors, in that order, from `gen`; a
    given x is used as is (nothing drawn for it)."""
    if x is None:
        x = torch.randn((lin.M, lin.K), generator=gen, dtype=torch.float32) * X_STD
        if outlier_fraction > 0.0:
            mask = torch.rand((lin.M, lin.K), generator=gen, dtype=torch.float32) < outlier_fraction
            x[mask] *= outlier_multiplier
            del mask
        x = x.to(torch.bfloat16)
    w = (torch.randn((lin.N, lin.K), generator=gen, dtype=torch.float32) * (1.0 / lin.K ** 0.5)).to(torch.bfloat16)
    dy = (torch.randn((lin.M, lin.N), generator=gen, dtype=torch.float32) * DY_STD).to(torch.bfloat16)
    return x, w, dy


def workload_inputs(wl: Workload, step: int = 0) -> List[Tuple[Linear, torch.Tensor, torch.Tensor, torch.Tensor]]:
    """All linears' (X, W, dY) for one step of a workload.  Dynamic workloads
    use `wl.seed`; delayed ones use a fresh seed per step (seed = step)."""
    seed = step if wl.scaling == "delayed" else wl.seed
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    out = []
    lead_x = {}
    for lin in wl.linears:
        group = next((g for g in wl.shared_x if lin.name in g), None)
        shared = lead_x.get(group) if group else None
        x, w, dy = draw_linear(gen, lin, wl.outlier_fraction, wl.outlier_multiplier, x=shared)
        if group and shared is None:
            lead_x[group] = x
        out.append((lin, x, w, dy))
    return out


def groups_of(wl: Workload):
    """Indices of wl.linears, grouped: one group per shared input (in order of
    first appearance), singletons otherwise."""
    groups, seen = [], {}
    for i, lin in enumerate(wl.linears):
        g = next((g for g in wl.shared_x if lin.name in g), None)
        if g is None:
            groups.append([i])
        elif g in seen:
            groups[seen[g]].append(i)
        else:
            seen[g] = len(groups)
            groups.append([i])
    return groups


def random_bf16(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    """A seeded N(0, std^2) bf16 CPU tensor for ad-hoc test shapes."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor):
    """The uint16 bit patterns of a bf16 CPU tensor, as a numpy array."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
