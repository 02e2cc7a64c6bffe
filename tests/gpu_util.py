"""Builders shared by the GPU tests: the same seeded weights feed the device
model (through the library's own W12 encoder) and the CPU oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle import model as om
from synth.configs import ModelConfig, gen_kv_context, gen_model
from synth.weights import bf16_bits_numpy


def build_pair(cfg: ModelConfig, seed: int, s_max: int, max_nodes: int = 64, gains: str = "random",
               device="cuda", with_hi8: bool = False):
    """Returns ``(device_model, oracle_model, oracle_cache)`` for ``cfg``."""
    from tree_verification_pass_amd.model import DeviceModel, Dims
    m = gen_model(cfg, seed, "cpu", gains)
    kv = [gen_kv_context(cfg, seed, layer, cfg.ctx_len, s_max) for layer in range(cfg.n_layers)]
    dev = torch.device(device)
    dm = DeviceModel(Dims.of(cfg), m.embed.to(dev), m.final_norm.to(dev), m.lm_head.to(dev),
                     lambda l: {k: v.to(dev) for k, v in m.layers[l].items()},
                     lambda l: (kv[l][0].to(dev), kv[l][1].to(dev)), s_max=s_max, max_nodes=max_nodes,
                     with_hi8=with_hi8)
    layers = [{k: bf16_bits_numpy(v) for k, v in layer.items()} for layer in m.layers]
    orc = om.OracleModel.from_bits(om.Dims.of(cfg), bf16_bits_numpy(m.embed), layers,
                                   bf16_bits_numpy(m.final_norm), bf16_bits_numpy(m.lm_head))
    cache = om.KVCache.from_bits([bf16_bits_numpy(k) for k, _ in kv], [bf16_bits_numpy(v) for _, v in kv])
    return dm, orc, cache


def to_i32(x, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def bits(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_numpy(t)
