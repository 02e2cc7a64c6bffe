"""Device-resident W12 target model: converts bf16 weights to W12, packs them
for the GEMM, owns the KV caches and the ``tvp_plan``.

The caller supplies the weights (any source: the synthetic generators in
tests and benchmarks); each tensor is converted by the library's own encoder
(``w12_encode_count`` + ``w12_encode``) and packer, then the bf16 copy is
dropped, so a 27B-like target never holds more than one layer in bf16.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import torch

from . import (TVP_CHAN_GATEUP, TVP_CHAN_PLAIN, TVP_CHAN_QKV, TVP_FMT_HI8, TVP_FMT_W12, PackedW12, Plan,
               TvpLayer, TvpModelDesc, W12Tensor, tvp_plan_create, w12_encode, w12_pack)


@dataclass(frozen=True)
class Dims:
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float = 1.0e6
    norm_eps: float = 1.0e-6

    @classmethod
    def of(cls, cfg) -> "Dims":
        return cls(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab,
                   cfg.rope_theta, cfg.norm_eps)


@dataclass
class DeviceLayer:
    wqkv: PackedW12
    wo: PackedW12
    wgu: PackedW12
    wdown: PackedW12
    attn_norm: torch.Tensor
    ffn_norm: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    canonical: Dict[str, W12Tensor] = field(default_factory=dict)
    hi8: Dict[str, PackedW12] = field(default_factory=dict)  # 8-bit leading views (Q pass), when built


def _pack(t: W12Tensor, name: str, dims: Dims, fmt: int) -> PackedW12:
    if name == "wqkv":
        return w12_pack(t, TVP_CHAN_QKV, dims.n_heads, dims.n_kv_heads, dims.head_dim, fmt=fmt)
    if name == "wgu":
        return w12_pack(t, TVP_CHAN_GATEUP, dims.ffn, fmt=fmt)
    return w12_pack(t, TVP_CHAN_PLAIN, fmt=fmt)


def pack_linear(w: torch.Tensor, name: str, dims: Dims, keep: Optional[Dict[str, W12Tensor]] = None,
                hi8: Optional[Dict[str, PackedW12]] = None) -> PackedW12:
    """W12-encode one bf16 ``[out, in]`` weight on the device and pack it with the
    channel map its fused epilogue needs (and, when ``hi8`` is given, a packed
    copy of its 8-bit leading view under the same name)."""
    t = w12_encode(w.contiguous())
    if keep is not None:
        keep[name] = t
    if hi8 is not None:
        hi8[name] = _pack(t, name, dims, TVP_FMT_HI8)
    return _pack(t, name, dims, TVP_FMT_W12)


class DeviceModel:
    """A target model resident on one GPU, ready for ``verify_step``.

    ``layer_fn(l)`` returns the bf16 tensors of layer ``l`` (``wqkv, wo, wgu,
    wdown, attn_norm, ffn_norm``) on the device; ``kv_fn(l)`` returns that
    layer's K and V caches ``[n_kv_heads, s_max, head_dim]`` (context filled).
    With ``with_hi8`` every weight also gets a packed copy of its 8-bit leading
    view, and ``q_plan`` is the plan of the Q pass of two-level verification
    (same embedding, norms and KV caches; up to 32 nodes).
    """

    def __init__(self, dims: Dims, embed: torch.Tensor, final_norm: torch.Tensor, lm_head: torch.Tensor,
                 layer_fn: Callable[[int], Dict[str, torch.Tensor]],
                 kv_fn: Callable[[int], tuple], s_max: int, max_nodes: int = 32,
                 keep_canonical: bool = False, with_hi8: bool = False):
        self.dims = dims
        self.s_max = s_max
        self.device = embed.device
        self.embed = embed.contiguous()
        self.final_norm = final_norm.contiguous()
        self.canonical_lm: Dict[str, W12Tensor] = {}
        self.hi8_lm: Dict[str, PackedW12] = {}
        self.lm_head = pack_linear(lm_head, "lm_head", dims, self.canonical_lm if keep_canonical else None,
                                   self.hi8_lm if with_hi8 else None)
        self.layers: List[DeviceLayer] = []
        for layer in range(dims.n_layers):
            src = layer_fn(layer)
            keep: Dict[str, W12Tensor] = {}
            hi8: Dict[str, PackedW12] = {}
            packed = {k: pack_linear(src[k], k, dims, keep if keep_canonical else None, hi8 if with_hi8 else None)
                      for k in ("wqkv", "wo", "wgu", "wdown")}
            kc, vc = kv_fn(layer)
            self.layers.append(DeviceLayer(packed["wqkv"], packed["wo"], packed["wgu"], packed["wdown"],
                                           src["attn_norm"].contiguous(), src["ffn_norm"].contiguous(),
                                           kc.contiguous(), vc.contiguous(), keep, hi8))
            del src
        self.plan = self._make_plan(max_nodes)
        self.q_plan = self._make_plan(min(max_nodes, 32), hi8=True) if with_hi8 else None

    def _make_plan(self, max_nodes: int, hi8: bool = False) -> Plan:
        d = self.dims
        arr = (TvpLayer * d.n_layers)()
        lm = self.hi8_lm["lm_head"] if hi8 else self.lm_head
        keep = [self.embed, self.final_norm, lm.blob]
        for i, L in enumerate(self.layers):
            w = L.hi8 if hi8 else {"wqkv": L.wqkv, "wo": L.wo, "wgu": L.wgu, "wdown": L.wdown}
            arr[i] = TvpLayer(w["wqkv"].desc, w["wo"].desc, w["wgu"].desc, w["wdown"].desc, L.attn_norm.data_ptr(),
                              L.ffn_norm.data_ptr(), L.k_cache.data_ptr(), L.v_cache.data_ptr())
            keep += [w["wqkv"].blob, w["wo"].blob, w["wgu"].blob, w["wdown"].blob, L.attn_norm, L.ffn_norm,
                     L.k_cache, L.v_cache]
        desc = TvpModelDesc(d.n_layers, d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab,
                            d.rope_theta, d.norm_eps, self.s_max, self.embed.data_ptr(),
                            self.final_norm.data_ptr(), lm.desc,
                            ctypes.cast(arr, ctypes.POINTER(TvpLayer)))
        return tvp_plan_create(desc, arr, max_nodes, keep)

    def stream_bytes(self, hi8: bool = False) -> int:
        """Packed bytes one pass streams (records, escapes and per-channel data),
        of the W12 copies or of the 8-bit views."""
        if hi8:
            return self.hi8_lm["lm_head"].stream_bytes() + sum(p.stream_bytes() for L in self.layers
                                                                for p in L.hi8.values())
        total = self.lm_head.stream_bytes()
        for L in self.layers:
            total += L.wqkv.stream_bytes() + L.wo.stream_bytes() + L.wgu.stream_bytes() + L.wdown.stream_bytes()
        return total
