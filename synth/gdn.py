"""Seeded inputs of the Gated DeltaNet layers of a hybrid target (random
draws only; the recurrence itself is not computed here).

Recipe, per layer and draft tree of n nodes:

* q, k ``[n, hk, dk]``: ``N(0, 1)`` draws scaled to unit L2 norm per head in
  fp32, then rounded to bf16 (the layer normalises q and k before the
  recurrence);
* v ``[n, hv, dv]``: ``N(0, 1)`` rounded to bf16;
* log decay g ``[n, hv]`` fp32: ``log(alpha)`` with alpha uniform in
  ``[alpha_lo, alpha_hi]`` (default 0.90 .. 0.999);
* write strength beta ``[n, hv]`` fp32: uniform in ``[0.05, 0.95]``;
* committed state ``[hv, dv, dk]`` fp32: ``N(0, state_std^2)`` (default 0.25),
  the magnitude a unit-key, unit-value state settles at under such decays.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Union

import torch

from .weights import bf16_from_f32, make_generator, sub_seed


@dataclass(frozen=True)
class GdnShape:
    hk: int = 8     # key heads (q and k)
    hv: int = 40    # value heads (state, v, output)
    dk: int = 128
    dv: int = 128


# Shapes of one recurrent layer of the hybrid stand-ins: the 27B-like hybrid
# (48 of 64 layers recurrent, hidden 5120 = 40 value heads x 128, key heads
# as the dense layers' kv heads) and a tiny one for the oracle's sizes.
GDN_SHAPES = {
    "27b_hybrid": GdnShape(8, 40, 128, 128),
    "tiny": GdnShape(2, 4, 128, 128),
}
GDN_LAYERS_27B_HYBRID = 48


@dataclass
class GdnInputs:
    q: torch.Tensor      # bf16 [n, hk, dk]
    k: torch.Tensor      # bf16 [n, hk, dk]
    v: torch.Tensor      # bf16 [n, hv, dv]
    g: torch.Tensor      # fp32 [n, hv]
    beta: torch.Tensor   # fp32 [n, hv]
    state: torch.Tensor  # fp32 [hv, dv, dk]


def _unit_rows(gen: torch.Generator, shape, device) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return bf16_from_f32(x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30))


def gen_gdn_inputs(seed: int, layer: int, n: int, shape: GdnShape, device: Union[str, torch.device] = "cpu",
                   alpha_lo: float = 0.90, alpha_hi: float = 0.999, state_std: float = 0.25) -> GdnInputs:
    """Inputs of one recurrent layer for an n-node tree (CPU torch generator
    streams; the tensors are moved to ``device`` afterwards)."""
    gen = make_generator(sub_seed(seed, 70, layer, n), "cpu")
    q = _unit_rows(gen, (n, shape.hk, shape.dk), "cpu")
    k = _unit_rows(gen, (n, shape.hk, shape.dk), "cpu")
    v = bf16_from_f32(torch.randn(n, shape.hv, shape.dv, generator=gen, dtype=torch.float32))
    alpha = alpha_lo + (alpha_hi - alpha_lo) * torch.rand(n, shape.hv, generator=gen, dtype=torch.float64)
    g = torch.log(alpha).to(torch.float32)
    beta = (0.05 + 0.9 * torch.rand(n, shape.hv, generator=gen, dtype=torch.float64)).to(torch.float32)
    state = (state_std * torch.randn(shape.hv, shape.dv, shape.dk, generator=gen, dtype=torch.float32))
    return GdnInputs(*(t.to(device) for t in (q, k, v, g, beta, state)))
