"""Seeded generators and the five synthetic workloads.

Shapes follow a 70B-class decoder layer (grouped-query QKV 8192->10240, O
8192->8192, gate/up 8192->28672, down 28672->8192), the scale the page talks
about (a 70B bf16 model of 140 GB with 14 fine-tuned variants; section
"Matematiksel temel" and the figure in "Sunum mimarisi").
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# (name, d_out, d_in) of the five linears of one 70B-shaped decoder layer.
LAYER_70B = (
    ("qkv", 10240, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    matrices: tuple            # ((name, d_out, d_in), ...)
    sigma: float               # std of W_base
    b: float | None            # Laplace scale of the deltas (None: per variant)
    alpha_mode: int            # 0 per matrix, 1 per row
    tokens: tuple              # token counts M exercised
    n_variants: int = 1
    layers: int = 1
    note: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "single_256x512": Workload(
        "single_256x512", 0, (("w", 256, 512),), 0.02, 1e-3, 0, (4,),
        note="one small linear, scalar alpha, M=4"),
    "proj_4096": Workload(
        "proj_4096", 2, (("w", 4096, 4096),), 0.02, 5e-4, 1, (1, 4, 16),
        note="Llama-style 4096x4096 projection, per-row alpha, decode M=1,4,16"),
    "layer70b_multi": Workload(
        "layer70b_multi", 3, LAYER_70B, 0.015, None, 1, (32,), n_variants=14,
        note="one 70B-shaped layer, 14 variants, b_v log-uniform [2e-4, 2e-3], "
             "M=32 Zipf(1.1) variant mix"),
    "layer70b_prefill": Workload(
        "layer70b_prefill", 4, LAYER_70B, 0.015, 1e-3, 0, (2048,),
        note="one 70B-shaped layer, one variant, per-matrix alpha, prefill M=2048"),
    "layer70b_decode": Workload(
        "layer70b_decode", 6, LAYER_70B, 0.015, 5e-4, 1, (1, 4, 16),
        note="one 70B-shaped layer, one variant, per-row alpha, decode M=1,4,16 "
             "(the projection's decode token counts at the layer's shapes)"),
    "stack70b_multi": Workload(
        "stack70b_multi", 5, LAYER_70B, 0.015, 5e-4, 1, (64,), n_variants=14,
        layers=80,
        note="80 70B-shaped layers resident, 14 variants, M=64 Zipf(1.1) mix"),
}


# Smallest u of the Laplace inverse CDF: -1/2 plus one float32 step there.
U_MIN = -0.5 + 2.0 ** -25


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor, as a host numpy array."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_base(d_out: int, d_in: int, sigma: float, gen: torch.Generator,
              device="cpu") -> torch.Tensor:
    """W_base ~ N(0, sigma), bf16."""
    w = torch.randn(d_out, d_in, generator=gen, device=device, dtype=torch.float32)
    w.mul_(sigma)
    return w.to(torch.bfloat16)


def draw_finetuned(w_base: torch.Tensor, b: float, gen: torch.Generator) -> torch.Tensor:
    """W_ft = bf16(float32(W_base) + Laplace(0, b)) with the Laplace draw taken
    by inverse CDF from u ~ U(-1/2, 1/2)."""
    u = torch.rand(w_base.shape, generator=gen, device=w_base.device,
                   dtype=torch.float32)
    u.sub_(0.5)
    # rand can return exactly 0: keep u inside (-1/2, 1/2), where the inverse
    # CDF is finite (the clamped end is a draw of about 16.6 b)
    u.clamp_(min=U_MIN)
    lap = torch.log1p(u.abs().mul_(-2.0)).mul_(-b).mul_(torch.sign(u))
    del u
    lap.add_(w_base.to(torch.float32))
    return lap.to(torch.bfloat16)


def draw_activations(m: int, d_in: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """x ~ N(0, 1), bf16, shape [m, d_in]."""
    return torch.randn(m, d_in, generator=gen, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def laplace_scales(n_variants: int, seed: int, lo=2e-4, hi=2e-3) -> list:
    """Per-variant Laplace scales b_v, log-uniform in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [float(v) for v in np.exp(rng.uniform(np.log(lo), np.log(hi), n_variants))]


def zipf_ids(m: int, n_variants: int, seed: int, s: float = 1.1) -> np.ndarray:
    """m variant ids from a Zipf(s) law truncated to n_variants ranks;
    id 0 is the most popular."""
    ranks = np.arange(1, n_variants + 1, dtype=np.float64)
    p = ranks ** -s
    p /= p.sum()
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice(n_variants, size=m, p=p).astype(np.int32)


def small_pair(d_out: int, d_in: int, sigma: float, b: float, seed: int, device="cpu"):
    """(W_base, W_ft) for one matrix from one seed, drawn in that order."""
    g = _gen(seed, device)
    w = draw_base(d_out, d_in, sigma, g, device)
    return w, draw_finetuned(w, b, g)


def generator(seed: int, device="cpu") -> torch.Generator:
    return _gen(seed, device)


# ----------------------------------------------------------------- layers
def variant_scales(wl: Workload) -> list:
    """Laplace scale of each variant: the workload's fixed b, or per-variant
    log-uniform draws in [2e-4, 2e-3] seeded by the workload seed."""
    if wl.b is not None:
        return [wl.b] * wl.n_variants
    return laplace_scales(wl.n_variants, wl.seed)


def draw_layer_bases(wl: Workload, gen: torch.Generator, device) -> list:
    """W_base of each matrix of one layer, in matrix order."""
    return [draw_base(d_out, d_in, wl.sigma, gen, device) for _, d_out, d_in in wl.matrices]


def iter_finetuned(bases: list, scales: list, gen: torch.Generator):
    """Yield (variant, matrix index, W_ft), variant-major, one temporary at a
    time, so the caller can compress and drop each before the next."""
    for v, b in enumerate(scales):
        for i, w in enumerate(bases):
            yield v, i, draw_finetuned(w, b, gen)


def draw_layer_inputs(wl: Workload, m: int, gen: torch.Generator, device) -> list:
    """One activation tensor per matrix of the layer.  QKV, gate and up read
    the same [m, 8192] input, O its own [m, 8192], down a [m, 28672] one."""
    names = [name for name, _, _ in wl.matrices]
    if names == [n for n, _, _ in LAYER_70B]:
        x_in = draw_activations(m, 8192, gen, device)
        x_o = draw_activations(m, 8192, gen, device)
        x_down = draw_activations(m, 28672, gen, device)
        return [x_in, x_o, x_in, x_in, x_down]
    return [draw_activations(m, d_in, gen, device) for _, _, d_in in wl.matrices]


# ----------------------------------------------------------------- stacks
def draw_stack_bases(wl: Workload, gen: torch.Generator, device) -> list:
    """W_base of every layer of a stack: stack[l][i] is matrix i of layer l,
    drawn layer by layer in matrix order."""
    return [draw_layer_bases(wl, gen, device) for _ in range(wl.layers)]


def iter_stack_finetuned(stack: list, scales: list, gen: torch.Generator):
    """Yield (layer, variant, matrix index, W_ft) layer-major, then variant,
    then matrix, one temporary at a time."""
    for l, bases in enumerate(stack):
        for v, b in enumerate(scales):
            for i, w in enumerate(bases):
                yield l, v, i, draw_finetuned(w, b, gen)


def draw_stack_inputs(wl: Workload, m: int, gen: torch.Generator, device) -> list:
    """Per-layer activations (x ~ N(0, 1) for every layer, as the layer
    inputs are drawn for one layer)."""
    return [draw_layer_inputs(wl, m, gen, device) for _ in range(wl.layers)]


# ----------------------------------------------------------------- merges
def draw_gaussian(rows: int, cols: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """float32 [rows, cols] ~ N(0, 1) (the start of an orthogonal iteration)."""
    return torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)


def draw_lowrank_checkpoint(w_base: torch.Tensor, rank: int, scale: float, b_noise: float,
                            gen: torch.Generator) -> torch.Tensor:
    """A fine-tuned checkpoint whose task vector is a planted rank-`rank`
    part plus Laplace(0, b_noise) noise: sum_j s_j a_j b_j^T with a_j, b_j
    ~ N(0, 1) and s_j = scale * (1 - j / (2 rank)) / sqrt(rank), j = 0..rank-1
    (so its element rms is about `scale` and its singular values stand well
    above the noise's), drawn in float32 and added to the base, then rounded
    to bf16.  The draw order is a, b, noise."""
    d_out, d_in = w_base.shape
    dev = w_base.device
    a = torch.randn(d_out, rank, generator=gen, device=dev, dtype=torch.float32)
    b = torch.randn(d_in, rank, generator=gen, device=dev, dtype=torch.float32)
    s = torch.tensor([scale * (1.0 - j / (2.0 * rank)) / rank ** 0.5 for j in range(rank)],
                     device=dev, dtype=torch.float32)
    u = (torch.rand(d_out, d_in, generator=gen, device=dev, dtype=torch.float32) - 0.5).clamp_(
        min=U_MIN)
    noise = -b_noise * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return (w_base.float() + (a * s) @ b.T + noise).to(torch.bfloat16)
