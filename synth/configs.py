"""Model shapes and weight recipes of the synthetic targets, and a seeded model generator.

All targets are dense decoder stacks: RMSNorm -> fused QKV -> tree attention
(GQA) -> O -> residual -> RMSNorm -> fused gate/up -> SwiGLU -> down ->
residual, then a final RMSNorm and an untied LM head.  Weights are random;
the architecture is the one named by each configuration.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Union

import torch

from .weights import (LinearRecipe, gen_linear_bf16, gen_normal_bf16, make_generator,
                      sub_seed)

# Tiny target: every weight N(0, 0.02), 1% zeros, 0.1% outliers x300.
TINY_RECIPE = LinearRecipe(sigma=0.02, zero_frac=0.01, outlier_frac=0.001, outlier_mult=300.0)
# Large targets (and the standalone GEMM shapes): per-channel sigma log-uniform
# in [0.005, 0.05], 1% zeros, 0.05% outliers x1000.
LARGE_RECIPE = LinearRecipe(sigma=None, sigma_lo=0.005, sigma_hi=0.05, zero_frac=0.01,
                            outlier_frac=0.0005, outlier_mult=1000.0)
EMBED_RECIPE = LinearRecipe(sigma=0.02, zero_frac=0.0, outlier_frac=0.0)


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    ctx_len: int
    n_nodes: int
    recipe: LinearRecipe = LARGE_RECIPE
    embed_recipe: LinearRecipe = EMBED_RECIPE
    rope_theta: float = 1.0e6
    norm_eps: float = 1.0e-6
    tree: str = "best_first"  # or "chain"

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def linear_shapes(self) -> Dict[str, tuple]:
        h, f = self.hidden, self.ffn
        return {
            "wqkv": (self.qkv_out, h),
            "wo": (h, self.n_heads * self.head_dim),
            "wgu": (2 * f, h),
            "wdown": (h, f),
        }

    def streamed_params(self) -> int:
        per_layer = sum(a * b for a, b in self.linear_shapes().values())
        return per_layer * self.n_layers + self.vocab * self.hidden

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, ModelConfig] = {
    "tiny": ModelConfig("tiny", n_layers=1, hidden=512, n_heads=8, n_kv_heads=8, head_dim=64,
                        ffn=1408, vocab=4096, ctx_len=256, n_nodes=8, recipe=TINY_RECIPE,
                        embed_recipe=TINY_RECIPE, tree="chain"),
    "4b": ModelConfig("4b", n_layers=36, hidden=2560, n_heads=32, n_kv_heads=8, head_dim=128,
                      ffn=9728, vocab=151936, ctx_len=2048, n_nodes=32),
    "27b": ModelConfig("27b", n_layers=64, hidden=5120, n_heads=40, n_kv_heads=8, head_dim=128,
                       ffn=17408, vocab=151936, ctx_len=4096, n_nodes=32),
    # Parity-test shapes: dimensions that are not multiples of the kernels' tiles.
    "ragged": ModelConfig("ragged", n_layers=2, hidden=1000, n_heads=6, n_kv_heads=2,
                          head_dim=64, ffn=1000, vocab=3000, ctx_len=300, n_nodes=13,
                          recipe=TINY_RECIPE, embed_recipe=TINY_RECIPE),
}

# Tensor indices used to derive per-tensor seeds.
_T_EMBED, _T_LAYER, _T_FINAL_NORM, _T_LM, _T_KV = 0, 1, 2, 3, 4
_L_QKV, _L_O, _L_GU, _L_DOWN, _L_ANORM, _L_FNORM = 0, 1, 2, 3, 4, 5


@dataclass
class ModelWeights:
    """bf16 tensors of one synthetic target (canonical ``[out, in]`` layout)."""

    cfg: ModelConfig
    embed: torch.Tensor
    layers: List[Dict[str, torch.Tensor]] = field(default_factory=list)
    final_norm: Optional[torch.Tensor] = None
    lm_head: Optional[torch.Tensor] = None


def _gain(seed: int, path, n: int, mode: str, device) -> torch.Tensor:
    if mode == "ones":
        return torch.ones(n, dtype=torch.bfloat16, device=device)
    g = make_generator(sub_seed(seed, *path), device)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32) * 0.1 + 1.0
    return x.to(torch.bfloat16)


def gen_layer(cfg: ModelConfig, seed: int, layer: int, device="cpu",
              gains: str = "ones") -> Dict[str, torch.Tensor]:
    out: Dict[str, torch.Tensor] = {}
    for j, (name, (n_out, k_in)) in enumerate(cfg.linear_shapes().items()):
        g = make_generator(sub_seed(seed, _T_LAYER, layer, j), device)
        out[name] = gen_linear_bf16(g, n_out, k_in, cfg.recipe, device=device)
    out["attn_norm"] = _gain(seed, (_T_LAYER, layer, _L_ANORM), cfg.hidden, gains, device)
    out["ffn_norm"] = _gain(seed, (_T_LAYER, layer, _L_FNORM), cfg.hidden, gains, device)
    return out


def gen_embed(cfg: ModelConfig, seed: int, device="cpu") -> torch.Tensor:
    g = make_generator(sub_seed(seed, _T_EMBED), device)
    return gen_linear_bf16(g, cfg.vocab, cfg.hidden, cfg.embed_recipe, device=device)


def gen_lm_head(cfg: ModelConfig, seed: int, device="cpu") -> torch.Tensor:
    g = make_generator(sub_seed(seed, _T_LM), device)
    return gen_linear_bf16(g, cfg.vocab, cfg.hidden, cfg.recipe, device=device)


def gen_final_norm(cfg: ModelConfig, seed: int, device="cpu", gains: str = "ones") -> torch.Tensor:
    return _gain(seed, (_T_FINAL_NORM,), cfg.hidden, gains, device)


def gen_model(cfg: ModelConfig, seed: int, device="cpu", gains: str = "ones") -> ModelWeights:
    m = ModelWeights(cfg=cfg, embed=gen_embed(cfg, seed, device))
    for layer in range(cfg.n_layers):
        m.layers.append(gen_layer(cfg, seed, layer, device, gains))
    m.final_norm = gen_final_norm(cfg, seed, device, gains)
    m.lm_head = gen_lm_head(cfg, seed, device)
    return m


def gen_kv_context(cfg: ModelConfig, seed: int, layer: int, ctx_len: int, s_max: int,
                   device: Union[str, torch.device] = "cpu"):
    """Committed context of one layer: K (already rotated) and V, ``N(0,1)`` bf16,
    returned in ``[kv_heads, s_max, head_dim]`` buffers whose first ``ctx_len``
    slots are filled (the rest zero)."""
    g = make_generator(sub_seed(seed, _T_KV, layer), device)
    k = torch.zeros(cfg.n_kv_heads, s_max, cfg.head_dim, dtype=torch.bfloat16, device=device)
    v = torch.zeros_like(k)
    if ctx_len > 0:
        k[:, :ctx_len] = gen_normal_bf16(g, (cfg.n_kv_heads, ctx_len, cfg.head_dim))
        v[:, :ctx_len] = gen_normal_bf16(g, (cfg.n_kv_heads, ctx_len, cfg.head_dim))
    return k, v
