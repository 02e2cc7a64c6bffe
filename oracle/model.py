"""Plain greedy inference of a dense decoder over a draft tree (oracle).

Source: SpecPilot summary (onedev.kr), section 무엇인가 ("what it is"): the
target model checks every drafted token in a single forward pass; section
무엇과 다른가: the pass returns the matched path and a bonus token; section
전제와 한계 ("assumptions and limits"): being lossless allows only near-tie
flips caused by a different floating-point reduction order (GEMM tiling, tree
attention), so the definition is ordinary bf16 greedy decoding.

Definition used here (the plainest reading of the pages): for every
tree node ``v`` the logits are the target's next-token logits after the
sequence ``context + tokens on the root-to-v path``, i.e. ordinary causal
attention along that path.  ``forward_tree`` computes all nodes in one pass
with an ancestor mask; ``verify_by_paths`` computes each node on its own by
token-at-a-time decoding and is the definition-level cross-check.

Architecture readings (the configurations name RMSNorm, RoPE, SwiGLU and
GQA only): RMSNorm ``x * (mean(x^2) + eps)^-1/2 * g``; RoPE rotate-half over
the whole head dimension with frequencies ``theta^(-2i/d)`` at position
``ctx_len + depth``; fused QKV rows ``[q heads | k heads | v heads]``; query
head ``h`` reads KV head ``h // (n_heads / n_kv_heads)``; fused gate/up rows
``[gate | up]``; ``silu(x) = x / (1 + exp(-x))``; no biases; untied LM head.

Rounding: values are bf16 at these points and fp64 everywhere in between:
``h = E[tokens]``; ``a = bf16(rmsnorm(h) * g1)``; ``q, k = bf16(rope(.))``,
``v = bf16(.)`` (k and v are what the cache stores); ``o = bf16(attention)``;
``h = bf16(h + o Wo^T)``; ``b = bf16(rmsnorm(h) * g2)``;
``u = bf16(silu(gate) * up)``; ``h = bf16(h + u Wd^T)``;
``f = bf16(rmsnorm(h) * g_f)``; logits ``f Wlm^T`` are not rounded.
"""

from __future__ import annotations

import copy
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import accept as _accept
from . import w12 as _w12
from .bf16 import from_bits, round_bf16


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
        return cls(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                   cfg.vocab, cfg.rope_theta, cfg.norm_eps)


class OracleModel:
    """Weights as fp64 arrays holding bf16 values."""

    def __init__(self, dims: Dims, embed: np.ndarray, layers: List[Dict[str, np.ndarray]],
                 final_norm: np.ndarray, lm_head: Optional[np.ndarray]):
        self.dims = dims
        self.embed = embed
        self.layers = layers
        self.final_norm = final_norm
        self.lm_head = lm_head

    @classmethod
    def from_bits(cls, dims: Dims, embed, layers, final_norm, lm_head) -> "OracleModel":
        """From raw bf16 bit patterns (uint16 arrays); ``layers`` holds dicts with
        ``wqkv, wo, wgu, wdown, attn_norm, ffn_norm``."""
        conv = [{k: from_bits(v) for k, v in layer.items()} for layer in layers]
        return cls(dims, from_bits(embed), conv, from_bits(final_norm),
                   None if lm_head is None else from_bits(lm_head))

    @classmethod
    def from_w12(cls, dims: Dims, embed, layers, final_norm, lm_head, view: str = "exact") -> "OracleModel":
        """From W12 tensors: every ``W12Tensor`` value is decoded exactly first
        (``view="exact"``), or through the 8-bit leading view of its records
        (``view="hi8"``, the Q pass of two-level verification, see
        ``w12.decode_hi8``)."""
        decode = {"exact": _w12.decode, "hi8": _w12.decode_hi8}[view]

        def dec(x):
            return from_bits(decode(x) if isinstance(x, _w12.W12Tensor) else x)
        conv = [{k: dec(v) for k, v in layer.items()} for layer in layers]
        return cls(dims, from_bits(embed), conv, from_bits(final_norm),
                   None if lm_head is None else dec(lm_head))


class KVCache:
    """Per-layer K and V, ``[n_kv_heads, s_max, head_dim]`` fp64 holding bf16 values."""

    def __init__(self, k: List[np.ndarray], v: List[np.ndarray]):
        self.k = k
        self.v = v

    @classmethod
    def from_bits(cls, ks, vs) -> "KVCache":
        return cls([from_bits(k) for k in ks], [from_bits(v) for v in vs])

    def copy(self) -> "KVCache":
        return KVCache([k.copy() for k in self.k], [v.copy() for v in self.v])


# ---------------------------------------------------------------- primitives

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    return theta ** (-(2.0 * np.arange(d // 2)) / d)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE; ``x`` is ``[n, heads, d]``, ``pos`` is ``[n]``."""
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """``q [n, hq, d]``, ``k, v [hkv, T, d]``, ``visible [n, T]`` -> ``[n, hq, d]``.

    Scores ``q.k / sqrt(d)``, masked softmax over the visible keys, weighted
    sum of values; query head ``h`` reads KV head ``h // (hq / hkv)``."""
    n, hq, d = q.shape
    hkv = k.shape[0]
    group = hq // hkv
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    for h in range(hq):
        kh = h // group
        s = (q[:, h, :] @ k[kh].T) * scale
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[kh]
    return out


def ancestor_mask(parents: Sequence[int]) -> np.ndarray:
    """``M[i, j]`` is true when node ``j`` is node ``i`` or one of its ancestors."""
    n = len(parents)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j != -1:
            m[i, j] = True
            j = parents[j]
    return m


# ------------------------------------------------------------------- forward

def layer_forward(model: OracleModel, layer: int, h: np.ndarray, pos: np.ndarray,
                  k_ctx: np.ndarray, v_ctx: np.ndarray, tree_visible: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One decoder layer over ``n`` new rows.

    ``k_ctx, v_ctx [hkv, L, d]`` are the committed keys/values (all visible),
    ``tree_visible [n, n]`` says which new rows each new row may attend to.
    Returns the new hidden rows and the rounded ``k, v [n, hkv, d]`` of the rows.
    """
    dm = model.dims
    w = model.layers[layer]
    n = h.shape[0]
    hq, hkv, d = dm.n_heads, dm.n_kv_heads, dm.head_dim
    a = round_bf16(rmsnorm(h, w["attn_norm"], dm.norm_eps))
    qkv = a @ w["wqkv"].T
    q = qkv[:, : hq * d].reshape(n, hq, d)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(n, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(n, hkv, d)
    q = round_bf16(rope(q, pos, dm.rope_theta))
    k = round_bf16(rope(k, pos, dm.rope_theta))
    v = round_bf16(v)
    keys = np.concatenate([k_ctx, k.transpose(1, 0, 2)], axis=1)
    vals = np.concatenate([v_ctx, v.transpose(1, 0, 2)], axis=1)
    L = k_ctx.shape[1]
    visible = np.concatenate([np.ones((n, L), dtype=bool), tree_visible], axis=1)
    o = round_bf16(attention(q, keys, vals, visible))
    h = round_bf16(h + o.reshape(n, hq * d) @ w["wo"].T)
    b = round_bf16(rmsnorm(h, w["ffn_norm"], dm.norm_eps))
    gu = b @ w["wgu"].T
    u = round_bf16(silu(gu[:, : dm.ffn]) * gu[:, dm.ffn:])
    h = round_bf16(h + u @ w["wdown"].T)
    return h, k, v


def final_hidden(model: OracleModel, h: np.ndarray) -> np.ndarray:
    return round_bf16(rmsnorm(h, model.final_norm, model.dims.norm_eps))


def lm_logits(model: OracleModel, f: np.ndarray) -> np.ndarray:
    return f @ model.lm_head.T


def forward_tree(model: OracleModel, cache: KVCache, ctx_len: int, tokens: Sequence[int],
                 parents: Sequence[int]):
    """All tree nodes in one pass.  Returns ``(logits [n, V], [(k, v)] per layer)``."""
    _accept.validate_tree(parents)
    tok = np.asarray(tokens, dtype=np.int64)
    pos = ctx_len + _accept.depths(parents)
    vis = ancestor_mask(parents)
    h = model.embed[tok]
    kv_new = []
    for layer in range(model.dims.n_layers):
        h, k, v = layer_forward(model, layer, h, pos, cache.k[layer][:, :ctx_len],
                                cache.v[layer][:, :ctx_len], vis)
        kv_new.append((k, v))
    return lm_logits(model, final_hidden(model, h)), kv_new


def greedy(logits: np.ndarray) -> np.ndarray:
    """Greedy token per row; ties go to the smallest token id."""
    return np.argmax(logits, axis=-1).astype(np.int64)


def verify(model: OracleModel, cache: KVCache, ctx_len: int, tokens: Sequence[int],
           parents: Sequence[int]) -> dict:
    logits, kv_new = forward_tree(model, cache, ctx_len, tokens, parents)
    am = greedy(logits)
    path, n_acc, bonus = _accept.accept(am, tokens, parents)
    return {"logits": logits, "argmax": am, "path": path, "n_accepted": n_acc,
            "bonus": bonus, "kv_new": kv_new}


def commit(cache: KVCache, ctx_len: int, path: Sequence[int], kv_new) -> int:
    """Write the accepted nodes' keys/values to slots ``ctx_len .. ctx_len + a``
    (root first) and return the new committed length ``ctx_len + a + 1``."""
    for layer, (k, v) in enumerate(kv_new):
        for j, node in enumerate(path):
            cache.k[layer][:, ctx_len + j] = k[node]
            cache.v[layer][:, ctx_len + j] = v[node]
    return ctx_len + len(path)


def decode_one(model: OracleModel, cache: KVCache, ctx_len: int, token: int) -> np.ndarray:
    """Single-token step at position ``ctx_len``: logits ``[V]``; appends its K/V
    to slot ``ctx_len`` of the cache."""
    h = model.embed[np.asarray([token], dtype=np.int64)]
    pos = np.asarray([ctx_len])
    self_only = np.ones((1, 1), dtype=bool)
    for layer in range(model.dims.n_layers):
        h, k, v = layer_forward(model, layer, h, pos, cache.k[layer][:, :ctx_len],
                                cache.v[layer][:, :ctx_len], self_only)
        cache.k[layer][:, ctx_len] = k[0]
        cache.v[layer][:, ctx_len] = v[0]
    return lm_logits(model, final_hidden(model, h))[0]


def verify_by_paths(model: OracleModel, cache: KVCache, ctx_len: int, tokens: Sequence[int],
                    parents: Sequence[int]) -> np.ndarray:
    """Definition-level logits: each node's root path decoded token by token."""
    _accept.validate_tree(parents)
    out = np.empty((len(parents), model.dims.vocab))
    for v in range(len(parents)):
        path = [v]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path.reverse()
        c = cache.copy()
        for j, node in enumerate(path):
            lg = decode_one(model, c, ctx_len + j, int(tokens[node]))
        out[v] = lg
    return out


def ar_greedy(model: OracleModel, cache: KVCache, ctx_len: int, root_token: int,
              n_tokens: int) -> List[int]:
    """``n_tokens`` greedy tokens after ``context + root_token`` (cache is copied)."""
    c = cache.copy()
    out: List[int] = []
    tok = int(root_token)
    for j in range(n_tokens):
        lg = decode_one(model, c, ctx_len + j, tok)
        tok = int(greedy(lg))
        out.append(tok)
    return out


def verify_batched(model: OracleModel, caches: List[KVCache], ctx_lens: Sequence[int],
                   tokens: Sequence[Sequence[int]], parents: Sequence[Sequence[int]]) -> List[dict]:
    """Requests sharing one pass are independent: each is its own verification."""
    return [verify(model, caches[r], int(ctx_lens[r]), tokens[r], parents[r])
            for r in range(len(caches))]
