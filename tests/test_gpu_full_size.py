"""The verification pass at full model shapes, in the launch configuration
bench.py times: the 27B-like shapes (hidden 5120, 40 query / 8 KV heads of
128, SwiGLU 17408, 4096-token context) and the 4B-like shapes (hidden 2560,
32 / 8 heads of 128, SwiGLU 9728, 2048-token context), each with the full
151936-token LM head and a 32-node best-first tree; and the batched pass at
the 27B-like shapes (24 requests sharing a 192-node budget, trees of 4-16
nodes, contexts uniform in [512, 8192]).  One decoder layer each (the
oracle's fp64 cost of a whole model would not fit a test).  Logits are compared on every row within max(2e-3, 1.5 x the
rounding-noise envelope of fp32 evaluations of the same definition, see
tests/fp32_reference.py), greedy tokens on decidable rows, acceptance where
determined; the pass is bitwise reproducible."""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.accept import accept as oaccept
from oracle.bf16 import from_bits
from synth import best_first_topology
from synth.configs import CONFIGS, gen_kv_context, gen_model
from synth.trees import assign_tokens_by_depth
from synth.weights import bf16_bits_numpy
from tests.fp32_reference import logit_tolerance, noise_envelope
from tests.gpu_util import to_i32
from tests.helpers import oracle_topk_fn
from tests.parity import acceptance_ok, check_logits

pytestmark = pytest.mark.gpu


class _Rows:
    """Embedding rows converted on demand (the full fp64 table would be 6 GB)."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits

    def __getitem__(self, idx):
        return from_bits(self.bits[idx])


@pytest.mark.parametrize("cfg_name", ["4b", "27b"])
def test_verify_step_full_shapes_one_layer(cuda, cfg_name):
    import tree_verification_pass_amd as tvp
    from tree_verification_pass_amd.model import DeviceModel, Dims

    cfg = dataclasses.replace(CONFIGS[cfg_name], n_layers=1)
    L, s_max, n = cfg.ctx_len, cfg.ctx_len + 64, cfg.n_nodes
    print(f"[full size] {cfg_name}: 1 layer, ctx {L}, {n} nodes, vocab {cfg.vocab}", flush=True)
    m = gen_model(cfg, 5, cuda, "random")
    kc, vc = gen_kv_context(cfg, 5, 0, L, s_max, device=cuda)
    dm = DeviceModel(Dims.of(cfg), m.embed, m.final_norm, m.lm_head, lambda l: m.layers[l],
                     lambda l: (kc, vc), s_max=s_max, max_nodes=n)
    layer_bits = {k: bf16_bits_numpy(v) for k, v in m.layers[0].items()}
    orc = om.OracleModel(om.Dims.of(cfg), _Rows(bf16_bits_numpy(m.embed)),
                         [{k: from_bits(v) for k, v in layer_bits.items()}],
                         from_bits(bf16_bits_numpy(m.final_norm)), from_bits(bf16_bits_numpy(m.lm_head)))
    cache = om.KVCache.from_bits([bf16_bits_numpy(kc)], [bf16_bits_numpy(vc)])
    rng = np.random.default_rng(6)
    parents, rank, _ = best_first_topology(rng, n)
    # draft tokens from the oracle's own top-4 at each parent, level by level
    tokens = assign_tokens_by_depth(rng, parents, rank, int(rng.integers(cfg.vocab)), cfg.vocab,
                                    oracle_topk_fn(orc, cache, L), 0.7)
    print("  oracle forward", flush=True)
    ref = om.verify(orc, cache, L, tokens, parents)
    print("  gpu pass", flush=True)
    res = tvp.verify_step(dm.plan, L, to_i32(tokens), to_i32(parents), commit=False, want_logits=True)
    res2 = tvp.verify_step(dm.plan, L, to_i32(tokens), to_i32(parents), commit=False, want_logits=True)
    torch.cuda.synchronize()
    g = res.logits.cpu().numpy().astype(np.float64)
    print("  rounding-noise envelope", flush=True)
    env = noise_envelope(orc, cache, L, tokens, parents, ref["logits"], runs=2)
    tol = logit_tolerance(env)
    chk = check_logits(g, ref["logits"], tol=tol)
    print(f"  logits max_abs_rel={chk['max_abs_rel']:.2e} fp32-envelope={env:.2e} tol={tol:.2e} "
          f"undecidable={chk['undecidable_frac']:.3f} accepted={int(res.n_accepted.item())} "
          f"(oracle {ref['n_accepted']})", flush=True)
    assert chk["logits_ok"], chk["max_abs_rel"]
    assert chk["argmax_ok"], chk["bad_argmax_rows"]
    am = res.argmax.cpu().numpy()
    assert np.array_equal(am, np.argmax(res.logits.cpu().numpy(), axis=1))
    p_own, a_own, b_own = oaccept(am, tokens, parents)
    assert int(res.n_accepted.item()) == a_own and int(res.bonus.item()) == b_own
    assert res.path.cpu().numpy()[: a_own + 1].tolist() == p_own
    assert acceptance_ok(am, ref["argmax"], tokens, parents, chk["decidable"])
    assert torch.equal(res.logits, res2.logits)


def test_verify_step_batched_27b_shapes_one_layer(cuda):
    """24 requests share a 192-node budget (trees of 4-16 nodes, best-first
    topology) over contexts uniform in [512, 8192], in one batched pass at the
    27B-like shapes.  Every request: status OK, argmax equal to the argmax of
    its own logits, acceptance following from its own greedy tokens, and the
    pass bitwise reproducible.  Six requests -- the shortest and longest
    context, the smallest and largest tree, one whose drafts come from the
    oracle's own top-4 and one more -- are compared with the oracle run on
    that request alone."""
    import tree_verification_pass_amd as tvp
    from synth.trees import batch_sizes
    from tree_verification_pass_amd.model import DeviceModel, Dims

    cfg = dataclasses.replace(CONFIGS["27b"], n_layers=1)
    n_req, ctx_lo, ctx_hi, cap = 24, 512, 8192, 16
    rng = np.random.default_rng(9)
    sizes = batch_sizes(rng, n_req=n_req, total=192, start=4, cap=cap)
    ctxs = rng.integers(ctx_lo, ctx_hi + 1, n_req)
    s_req = ctx_hi + cap
    s_max = n_req * s_req
    print(f"[full size] batched: {n_req} requests, {int(sizes.sum())} nodes, ctx {ctxs.min()}..{ctxs.max()}",
          flush=True)
    m = gen_model(cfg, 11, cuda, "random")
    kc = torch.zeros(cfg.n_kv_heads, s_max, cfg.head_dim, dtype=torch.bfloat16, device=cuda)
    vc = torch.zeros_like(kc)
    for r in range(n_req):  # request r owns slots [r * s_req, (r + 1) * s_req)
        k_r, v_r = gen_kv_context(cfg, 11, r, int(ctxs[r]), int(ctxs[r]), device=cuda)
        kc[:, r * s_req: r * s_req + ctxs[r]] = k_r
        vc[:, r * s_req: r * s_req + ctxs[r]] = v_r
    dm = DeviceModel(Dims.of(cfg), m.embed, m.final_norm, m.lm_head, lambda l: m.layers[l],
                     lambda l: (kc, vc), s_max=s_max, max_nodes=int(sizes.sum()))
    layer_bits = {k: bf16_bits_numpy(v) for k, v in m.layers[0].items()}
    orc = om.OracleModel(om.Dims.of(cfg), _Rows(bf16_bits_numpy(m.embed)),
                         [{k: from_bits(v) for k, v in layer_bits.items()}],
                         from_bits(bf16_bits_numpy(m.final_norm)), from_bits(bf16_bits_numpy(m.lm_head)))

    def cache_of(r):
        sl = slice(r * s_req, r * s_req + int(ctxs[r]))
        return om.KVCache.from_bits([bf16_bits_numpy(kc[:, sl])], [bf16_bits_numpy(vc[:, sl])])

    sampled = sorted({int(np.argmin(ctxs)), int(np.argmax(ctxs)), int(np.argmin(sizes)), int(np.argmax(sizes))})
    extra = [r for r in range(n_req) if r not in sampled]
    drafted = extra[0]
    sampled = sorted(set(sampled) | {drafted, extra[len(extra) // 2]})
    trees, toks = [], []
    for r in range(n_req):
        parents, rank, _ = best_first_topology(rng, int(sizes[r]))
        if r == drafted:
            tokens = assign_tokens_by_depth(rng, parents, rank, int(rng.integers(cfg.vocab)), cfg.vocab,
                                            oracle_topk_fn(orc, cache_of(r), int(ctxs[r])), 0.7)
        else:
            tokens = rng.integers(0, cfg.vocab, int(sizes[r])).astype(np.int32)
        trees.append(np.asarray(parents, np.int32))
        toks.append(np.asarray(tokens, np.int32))
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T, P = to_i32(np.concatenate(toks)), to_i32(np.concatenate(trees))
    print("  gpu pass", flush=True)
    res = tvp.verify_step_batched(dm.plan, ctxs.tolist(), node_ptr.tolist(), s_req, T, P, commit=False,
                                  want_logits=True)
    res2 = tvp.verify_step_batched(dm.plan, ctxs.tolist(), node_ptr.tolist(), s_req, T, P, commit=False,
                                   want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(res.logits, res2.logits) and torch.equal(res.argmax, res2.argmax)
    lg_dev = res.logits
    am_all = res.argmax.cpu().numpy()
    assert np.array_equal(am_all, torch.argmax(lg_dev, dim=1).cpu().numpy())
    path_all = res.path.cpu().numpy()
    for r in range(n_req):
        sl = slice(node_ptr[r], node_ptr[r + 1])
        p_own, a_own, b_own = oaccept(am_all[sl], toks[r], trees[r])
        assert int(res.status[r].item()) == 0
        assert int(res.n_accepted[r].item()) == a_own and int(res.bonus[r].item()) == b_own
        assert path_all[sl][: a_own + 1].tolist() == p_own
    for r in sampled:
        sl = slice(node_ptr[r], node_ptr[r + 1])
        cache = cache_of(r)
        ref = om.verify(orc, cache, int(ctxs[r]), toks[r], trees[r])
        env = noise_envelope(orc, cache, int(ctxs[r]), toks[r], trees[r], ref["logits"], runs=1)
        chk = check_logits(lg_dev[sl].cpu().numpy().astype(np.float64), ref["logits"], tol=logit_tolerance(env))
        print(f"  request {r}: {sizes[r]} nodes, ctx {ctxs[r]}: max_abs_rel={chk['max_abs_rel']:.2e} "
              f"envelope={env:.2e} accepted={int(res.n_accepted[r].item())} (oracle {ref['n_accepted']})",
              flush=True)
        assert chk["logits_ok"] and chk["argmax_ok"], (r, chk["max_abs_rel"], env)
        assert acceptance_ok(am_all[sl], ref["argmax"], toks[r], trees[r], chk["decidable"])
