"""Test helpers: build oracle models and caches from the synthetic generators."""

from __future__ import annotations

import numpy as np

from oracle import model as om
from oracle import w12
from synth.configs import ModelConfig, gen_kv_context, gen_model
from synth.weights import bf16_bits_numpy

LINEAR = ("wqkv", "wo", "wgu", "wdown")


def model_bits(cfg: ModelConfig, seed: int, gains: str = "random"):
    m = gen_model(cfg, seed, "cpu", gains)
    layers = [{k: bf16_bits_numpy(v) for k, v in layer.items()} for layer in m.layers]
    return (bf16_bits_numpy(m.embed), layers, bf16_bits_numpy(m.final_norm),
            bf16_bits_numpy(m.lm_head))


def oracle_model(cfg: ModelConfig, seed: int, gains: str = "random", via_w12: bool = True):
    embed, layers, fnorm, lm = model_bits(cfg, seed, gains)
    dims = om.Dims.of(cfg)
    if via_w12:
        enc = [{k: (w12.encode(v) if k in LINEAR else v) for k, v in layer.items()}
               for layer in layers]
        return om.OracleModel.from_w12(dims, embed, enc, fnorm, w12.encode(lm))
    return om.OracleModel.from_bits(dims, embed, layers, fnorm, lm)


def oracle_cache(cfg: ModelConfig, seed: int, ctx_len: int, s_max: int) -> om.KVCache:
    ks, vs = [], []
    for layer in range(cfg.n_layers):
        k, v = gen_kv_context(cfg, seed, layer, ctx_len, s_max)
        ks.append(bf16_bits_numpy(k))
        vs.append(bf16_bits_numpy(v))
    return om.KVCache.from_bits(ks, vs)


def oracle_topk_fn(model: om.OracleModel, cache: om.KVCache, ctx_len: int, k: int = 4):
    def fn(tokens, parents):
        logits, _ = om.forward_tree(model, cache, ctx_len, tokens, parents)
        return np.argsort(-logits, axis=1, kind="stable")[:, :k]
    return fn
