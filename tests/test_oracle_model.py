"""Pins for the oracle forward pass and verification.

Library equivalences: RMSNorm (torch rms_norm), attention with GQA (torch
scaled_dot_product_attention), SiLU, RoPE as complex rotation; a full layer
rebuilt from those library routines.  Definitions: the one-pass tree forward
equals token-by-token decoding of every root path; a chain of the greedy
continuation is accepted in full; a speculative loop emits the greedy stream.
Negative test: the fault model of the SpecPilot summary (section 전제와 한계:
logit bias +2 on every 7th vocabulary id after 2048 tokens) is rejected by the
parity checker.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from oracle.bf16 import round_bf16
from synth import best_first_topology, chain_topology
from synth.configs import CONFIGS, ModelConfig, TINY_RECIPE
from synth.trees import assign_tokens_by_depth
from tests.helpers import oracle_cache, oracle_model, oracle_topk_fn
from tests.parity import acceptance_ok, check_logits

SMALL = ModelConfig("small", n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                    vocab=50, ctx_len=5, n_nodes=6, recipe=TINY_RECIPE, embed_recipe=TINY_RECIPE)


def test_rope_pins():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 16))
    assert np.allclose(om.rope(x, np.zeros(5), 1e6), x, atol=0, rtol=0)
    pos = rng.integers(0, 9000, 5)
    y = om.rope(x, pos, 1e6)
    # rotation preserves the norm of every (i, i + d/2) pair
    assert np.allclose(x[..., :8] ** 2 + x[..., 8:] ** 2, y[..., :8] ** 2 + y[..., 8:] ** 2)
    # complex form: (x_i + j x_{i+d/2}) * exp(j * pos * theta^(-2i/d))
    xc = torch.complex(torch.from_numpy(x[..., :8]), torch.from_numpy(x[..., 8:]))
    inv = 1e6 ** (-(2.0 * torch.arange(8, dtype=torch.float64)) / 16)
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
    rot = xc * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    assert np.allclose(y, torch.cat([rot.real, rot.imag], dim=-1).numpy(), atol=1e-12)
    # scores depend on the position difference only
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    s1 = np.sum(om.rope(q, np.array([100]), 1e4) * om.rope(k, np.array([37]), 1e4))
    s2 = np.sum(om.rope(q, np.array([1063]), 1e4) * om.rope(k, np.array([1000]), 1e4))
    assert abs(s1 - s2) < 1e-9


def test_rmsnorm_and_silu_pins():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 40))
    g = rng.standard_normal(40)
    ref = F.rms_norm(torch.from_numpy(x), (40,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(om.rmsnorm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-12)
    c = np.full((1, 8), -3.0)
    assert np.allclose(om.rmsnorm(c, np.ones(8), 0.0), -1.0)
    z = np.linspace(-30, 30, 101)
    assert np.allclose(om.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-12, atol=1e-300)
    assert om.silu(np.array([0.0]))[0] == 0.0


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(2)
    n, hq, hkv, d, T = 6, 8, 2, 16, 11
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((hkv, T, d))
    v = rng.standard_normal((hkv, T, d))
    vis = rng.random((n, T)) < 0.6
    vis[:, 0] = True
    out = om.attention(q, k, v, vis)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=torch.from_numpy(vis), enable_gqa=True)
    assert np.allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def _torch_layer(w, h, pos, kctx, vctx, cfg):
    """One decoder layer from torch library routines (fp64), causal chain."""
    bf = lambda t: t.to(torch.bfloat16).to(torch.float64)  # noqa: E731
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    n, H = h.shape
    hq, hkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    h = T(h)
    a = bf(F.rms_norm(h, (H,), weight=T(w["attn_norm"]), eps=cfg.norm_eps))
    qkv = F.linear(a, T(w["wqkv"]))
    q = qkv[:, : hq * d].reshape(n, hq, d)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(n, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(n, hkv, d)
    inv = cfg.rope_theta ** (-(2.0 * torch.arange(d // 2, dtype=torch.float64)) / d)
    ang = T(pos)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(x):
        c = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot
        return torch.cat([c.real, c.imag], dim=-1)

    q, k, v = bf(rope(q)), bf(rope(k)), bf(v)
    K = torch.cat([T(kctx), k.permute(1, 0, 2)], dim=1)
    V = torch.cat([T(vctx), v.permute(1, 0, 2)], dim=1)
    L = kctx.shape[1]
    mask = torch.ones(n, L + n, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], K[None], V[None], attn_mask=mask,
                                       enable_gqa=True)[0].permute(1, 0, 2).reshape(n, hq * d)
    h = bf(h + F.linear(bf(o), T(w["wo"])))
    b = bf(F.rms_norm(h, (H,), weight=T(w["ffn_norm"]), eps=cfg.norm_eps))
    gu = F.linear(b, T(w["wgu"]))
    u = bf(F.silu(gu[:, : cfg.ffn]) * gu[:, cfg.ffn:])
    return bf(h + F.linear(u, T(w["wdown"]))).numpy()


def test_layer_matches_library_composition():
    m = oracle_model(SMALL, 3)
    cache = oracle_cache(SMALL, 3, SMALL.ctx_len, 32)
    rng = np.random.default_rng(4)
    n = 6
    tokens = rng.integers(0, SMALL.vocab, n)
    h0 = m.embed[tokens]
    pos = SMALL.ctx_len + np.arange(n)
    kc, vc = cache.k[0][:, : SMALL.ctx_len], cache.v[0][:, : SMALL.ctx_len]
    h1, _, _ = om.layer_forward(m, 0, h0, pos, kc, vc, np.tril(np.ones((n, n), dtype=bool)))
    ref = _torch_layer(m.layers[0], h0, pos, kc, vc, SMALL)
    # both sides round to bf16 at the same points; fp64 reduction order differs,
    # so allow a rare one-ulp bf16 difference
    diff = np.abs(h1 - ref)
    assert np.mean(diff == 0) > 0.99
    assert np.all(diff <= 2.0 ** -7 * np.maximum(np.abs(ref), 1e-30) + 1e-30)


@pytest.mark.parametrize("cfg_name,seed", [("small", 5), ("tiny", 0)])
def test_tree_pass_equals_path_by_path_decoding(cfg_name, seed):
    cfg = SMALL if cfg_name == "small" else CONFIGS["tiny"]
    m = oracle_model(cfg, seed)
    ctx = cfg.ctx_len
    cache = oracle_cache(cfg, seed, ctx, ctx + 16)
    rng = np.random.default_rng(seed)
    parents, _, _ = best_first_topology(rng, 8, max_branch=3, max_depth=4)
    tokens = rng.integers(0, cfg.vocab, 8)
    res = om.verify(m, cache, ctx, tokens, parents)
    ref = om.verify_by_paths(m, cache, ctx, tokens, parents)
    assert np.allclose(res["logits"], ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_chain_of_greedy_continuation_is_accepted():
    cfg = CONFIGS["tiny"]
    m = oracle_model(cfg, 0)
    cache = oracle_cache(cfg, 0, cfg.ctx_len, cfg.ctx_len + 16)
    root = 17
    ar = om.ar_greedy(m, cache, cfg.ctx_len, root, 8)
    tokens = [root] + ar[:7]
    res = om.verify(m, cache, cfg.ctx_len, tokens, chain_topology(8))
    assert res["n_accepted"] == 7 and res["bonus"] == ar[7]
    assert res["path"] == list(range(8))
    for j in range(1, 8):
        bad = list(tokens)
        bad[j] = (bad[j] + 1) % cfg.vocab
        r = om.verify(m, cache, cfg.ctx_len, bad, chain_topology(8))
        assert r["n_accepted"] == j - 1 and r["bonus"] == ar[j - 1]


def test_speculative_loop_emits_greedy_stream():
    cfg = SMALL
    m = oracle_model(cfg, 9)
    ctx0 = cfg.ctx_len
    cache = oracle_cache(cfg, 9, ctx0, 64)
    ref_stream = om.ar_greedy(m, cache, ctx0, 3, 30)
    rng = np.random.default_rng(9)
    ctx, root, stream = ctx0, 3, []
    while len(stream) < 30:
        parents, rank, _ = best_first_topology(rng, 6, max_depth=4)
        tokens = assign_tokens_by_depth(rng, parents, rank, root, cfg.vocab,
                                        oracle_topk_fn(m, cache, ctx), p_top=0.8)
        res = om.verify(m, cache, ctx, tokens, parents)
        stream += [int(tokens[i]) for i in res["path"][1:]] + [res["bonus"]]
        ctx = om.commit(cache, ctx, res["path"], res["kv_new"])
        root = res["bonus"]
    assert stream[:30] == ref_stream


def test_fault_injection_is_rejected():
    # The faulty system of the fault model: +2 on every 7th vocabulary id once
    # the position reaches 2048.  Planted in the oracle's output on the CPU.
    cfg = CONFIGS["tiny"].with_(ctx_len=2048)
    m = oracle_model(cfg, 1)
    cache = oracle_cache(cfg, 1, 2048, 2064)
    rng = np.random.default_rng(1)
    parents, _, _ = best_first_topology(rng, 8)
    tokens = rng.integers(0, cfg.vocab, 8)
    good = om.verify(m, cache, 2048, tokens, parents)
    bias = np.zeros(cfg.vocab)
    bias[::7] = 2.0
    faulty = good["logits"] + bias[None, :]
    ok = check_logits(good["logits"], good["logits"])
    assert ok["logits_ok"] and ok["argmax_ok"]
    bad = check_logits(faulty, good["logits"])
    assert not bad["logits_ok"]
    # every row whose greedy token the bias flips is a decidable mismatch
    # (its error, 2.0, exceeds the oracle's margin only by flipping)
    am_f = np.argmax(faulty, axis=1)
    flipped = np.flatnonzero(am_f != good["argmax"])
    assert set(flipped.tolist()) <= set(bad["bad_argmax_rows"]) | set(
        np.flatnonzero(~bad["decidable"]).tolist())
    assert bad["max_abs_rel"] > 10 * 2e-3
