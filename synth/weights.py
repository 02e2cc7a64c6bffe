"""Seeded weight, activation and KV-context generators (random draws only)."""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Union

import numpy as np
import torch

# Rows drawn per chunk.  Part of the recipe: the stream of draws depends on it.
ROW_CHUNK = 4096


def make_generator(seed: int, device: Union[str, torch.device] = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def sub_seed(seed: int, *path: int) -> int:
    """A 63-bit seed for one tensor, derived from the workload seed and an index path."""
    ss = np.random.SeedSequence([int(seed)] + [int(p) for p in path])
    lo, hi = ss.generate_state(2, dtype=np.uint32)
    return int((int(hi) << 31) ^ int(lo)) & ((1 << 63) - 1)


def bf16_from_f32(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 with torch's round-to-nearest-even conversion."""
    return x.to(torch.float32).to(torch.bfloat16)


def gen_normal_bf16(gen: torch.Generator, shape, std: float = 1.0,
                    device: Optional[Union[str, torch.device]] = None) -> torch.Tensor:
    dev = device if device is not None else gen.device
    x = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return bf16_from_f32(x)


def gen_sigmas_loguniform(gen: torch.Generator, n: int, lo: float, hi: float) -> torch.Tensor:
    u = torch.rand(n, generator=gen, device=gen.device, dtype=torch.float64)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.float32)


@dataclass(frozen=True)
class LinearRecipe:
    """Distribution of one linear weight tensor ``[n_out, k_in]``.

    ``sigma`` is a fixed standard deviation, or ``None`` to draw one per
    output channel log-uniformly in ``[sigma_lo, sigma_hi]``.
    """

    sigma: Optional[float] = 0.02
    sigma_lo: float = 0.005
    sigma_hi: float = 0.05
    zero_frac: float = 0.01
    outlier_frac: float = 0.001
    outlier_mult: float = 300.0


def gen_linear_bf16(gen: torch.Generator, n_out: int, k_in: int, recipe: LinearRecipe,
                    device: Optional[Union[str, torch.device]] = None) -> torch.Tensor:
    """bf16 weights ``[n_out, k_in]`` drawn by ``recipe``.

    Per channel, ``round(zero_frac*k_in)`` positions become exact +0.0 and the
    next ``round(outlier_frac*k_in)`` positions of the same seeded random order
    are multiplied by ``outlier_mult`` (so zeros and outliers are disjoint).
    """
    dev = torch.device(device) if device is not None else gen.device
    if recipe.sigma is None:
        sig = gen_sigmas_loguniform(gen, n_out, recipe.sigma_lo, recipe.sigma_hi).to(dev)
    else:
        sig = None
    nz = int(round(recipe.zero_frac * k_in))
    no = int(round(recipe.outlier_frac * k_in))
    out = torch.empty((n_out, k_in), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, n_out, ROW_CHUNK):
        r1 = min(n_out, r0 + ROW_CHUNK)
        rows = r1 - r0
        w = torch.randn(rows, k_in, generator=gen, device=dev, dtype=torch.float32)
        if sig is None:
            w.mul_(recipe.sigma)
        else:
            w.mul_(sig[r0:r1, None])
        if nz + no > 0:
            keys = torch.rand(rows, k_in, generator=gen, device=dev, dtype=torch.float32)
            idx = torch.topk(keys, nz + no, dim=1, largest=True, sorted=True).indices
            del keys
            if no > 0:
                oi = idx[:, nz:]
                w.scatter_(1, oi, torch.gather(w, 1, oi) * recipe.outlier_mult)
            if nz > 0:
                w.scatter_(1, idx[:, :nz], 0.0)
        out[r0:r1] = bf16_from_f32(w)
        del w
    return out


def bf16_bits_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as a host ``uint16`` array."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
