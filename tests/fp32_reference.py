"""Rounding-noise envelope of the verification pass.

With bf16 rounding points inside the pass, an fp32-accumulated value that
lands on the other side of a bf16 rounding boundary than the fp64 oracle's
flips one ulp, and on weights with large outliers a single flip can move a
logit by a few 1e-3 of the row maximum.  Two independent estimates of that
noise, both computed from the oracle's definition alone:

* ``forward_fp32``: an fp32 evaluation from torch CPU library routines, with a
  seeded permutation of every matmul's summation order;
* ``noisy_oracle``: the oracle itself with every value perturbed by a random
  relative amount of at most ``eta`` (fp32-accumulation level) just before
  each bf16 rounding point.

The end-to-end logit comparison is per row: row v may deviate by
max(2e-3, 1.5 x row v's envelope), never more than ROW_TOL_CAP (see
tests/parity.py); the kernel-level parity tests, which see identical inputs,
keep the plain bound.
"""

from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

from oracle import model as om


def forward_fp32(m: om.OracleModel, cache: om.KVCache, L: int, tokens, parents, seed: int = 0) -> np.ndarray:
    d = m.dims
    g = torch.Generator().manual_seed(seed)
    bf = lambda t: t.to(torch.bfloat16).to(torch.float32)  # noqa: E731
    T = lambda a: torch.from_numpy(np.asarray(a)).to(torch.float32)  # noqa: E731

    def mm(x, w):  # x [n, k] @ w[out, k]^T with a random summation order
        p = torch.randperm(x.shape[1], generator=g)
        return x[:, p] @ w[:, p].T

    n = len(tokens)
    hq, hkv, hd = d.n_heads, d.n_kv_heads, d.head_dim
    pos = L + om._accept.depths(parents)
    vis = torch.from_numpy(np.concatenate([np.ones((n, L), bool), om.ancestor_mask(parents)], 1))
    h = T(m.embed[np.asarray(tokens)])
    inv = torch.from_numpy(d.rope_theta ** (-(2.0 * np.arange(hd // 2)) / hd))
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None]
    c, s = torch.cos(ang).float()[:, None], torch.sin(ang).float()[:, None]

    def rope(x):
        x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
        return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], -1)

    for li, w in enumerate(m.layers):
        a = bf(F.rms_norm(h, (d.hidden,), weight=T(w["attn_norm"]), eps=d.norm_eps))
        qkv = mm(a, T(w["wqkv"]))
        q = bf(rope(qkv[:, : hq * hd].reshape(n, hq, hd)))
        k = bf(rope(qkv[:, hq * hd: (hq + hkv) * hd].reshape(n, hkv, hd)))
        v = bf(qkv[:, (hq + hkv) * hd:].reshape(n, hkv, hd))
        K = torch.cat([T(cache.k[li][:, :L]), k.permute(1, 0, 2)], 1)
        V = torch.cat([T(cache.v[li][:, :L]), v.permute(1, 0, 2)], 1)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], K[None], V[None], attn_mask=vis,
                                           enable_gqa=True)[0].permute(1, 0, 2)
        h = bf(h + mm(bf(o).reshape(n, -1), T(w["wo"])))
        b = bf(F.rms_norm(h, (d.hidden,), weight=T(w["ffn_norm"]), eps=d.norm_eps))
        gu = mm(b, T(w["wgu"]))
        u = bf(F.silu(gu[:, : d.ffn]) * gu[:, d.ffn:])
        h = bf(h + mm(u, T(w["wdown"])))
    f = bf(F.rms_norm(h, (d.hidden,), weight=T(m.final_norm), eps=d.norm_eps))
    return mm(f, T(m.lm_head)).double().numpy()


def noisy_oracle(m, cache, L, tokens, parents, seed: int, eta: float = 2.0 ** -18) -> np.ndarray:
    """Oracle logits with each pre-rounding value scaled by (1 + u), |u| <= eta."""
    from oracle import bf16 as obf

    rng = np.random.default_rng(seed)
    orig = om.round_bf16

    def noisy(x):
        x = np.asarray(x, dtype=np.float64)
        return obf.round_bf16(x * (1.0 + eta * (2.0 * rng.random(x.shape) - 1.0)))

    om.round_bf16 = noisy
    try:
        return om.forward_tree(m, cache, L, tokens, parents)[0]
    finally:
        om.round_bf16 = orig


def noise_envelope_rows(m, cache, L, tokens, parents, ref_logits: np.ndarray, runs: int = 4) -> np.ndarray:
    """Per logits row, the largest max-abs-rel deviation from the fp64 oracle
    over `runs` fp32 evaluations with different summation orders and `runs`
    noisy-rounding oracle evaluations."""
    from tests.parity import row_max_abs_rel
    worst = np.zeros(ref_logits.shape[0])
    for s in range(runs):
        for g in (forward_fp32(m, cache, L, tokens, parents, seed=1000 + s),
                  noisy_oracle(m, cache, L, tokens, parents, seed=2000 + s)):
            worst = np.maximum(worst, row_max_abs_rel(g, ref_logits))
    return worst
