"""The verification pass at full model shapes, in the launch configuration
bench.py times: the 27B-like shapes (hidden 5120, 40 query / 8 KV heads of
128, SwiGLU 17408, 4096-token context) and the 4B-like shapes (hidden 2560,
32 / 8 heads of 128, SwiGLU 9728, 2048-token context), each with the full
151936-token LM head and a 32-node best-first tree: one decoder layer of
each, and the whole 36-layer 4B-like target; and the batched pass at the
27B-like shapes (24 requests sharing a 192-node budget, trees of 4-16 nodes,
contexts uniform in [512, 8192]), every request compared.  Logits are
compared row by row within max(2e-3, 1.5 x the row's rounding-noise envelope
of fp32 evaluations of the same definition, see tests/fp32_reference.py),
at most ROW_TOL_CAP; greedy tokens on decidable rows, acceptance where
determined; the pass is bitwise reproducible."""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.accept import accept as oaccept
from oracle.bf16 import from_bits
from synth import best_first_topology
from synth.configs import CONFIGS, gen_kv_context, gen_layer, gen_model
from synth.trees import assign_tokens_by_depth
from synth.weights import bf16_bits_numpy
from tests.fp32_reference import noise_envelope_rows
from tests.gpu_util import to_i32
from tests.helpers import oracle_topk_fn
from tests.parity import acceptance_ok, check_logits, row_report, row_tolerances

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
    env = noise_envelope_rows(orc, cache, L, tokens, parents, ref["logits"], runs=3)
    tol = row_tolerances(env)
    chk = check_logits(g, ref["logits"], tol=tol)
    print(f"  logits {row_report(chk, env, tol)} accepted={int(res.n_accepted.item())} "
          f"(oracle {ref['n_accepted']})", flush=True)
    assert chk["logits_ok"], (chk["bad_rows"], chk["max_abs_rel"])
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
    pass bitwise reproducible.  Every request is compared with the oracle run
    on that request alone; two of them (the shortest and the longest
    context) carry drafts from the oracle's own top-4, so some of their
    drafts are accepted."""
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

    drafted = {int(np.argmin(ctxs)), int(np.argmax(ctxs))}
    trees, toks = [], []
    for r in range(n_req):
        parents, rank, _ = best_first_topology(rng, int(sizes[r]))
        if r in drafted:
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
    # the oracle and its rounding-noise envelope per request; one bound for the
    # whole batch, from the envelope pooled over every request's rows
    refs, envs = [], []
    for r in range(n_req):
        cache = cache_of(r)
        refs.append(om.verify(orc, cache, int(ctxs[r]), toks[r], trees[r]))
        envs.append(noise_envelope_rows(orc, cache, int(ctxs[r]), toks[r], trees[r], refs[r]["logits"], runs=1))
    tol_all = row_tolerances(np.concatenate(envs))
    above = []
    for r in range(n_req):
        sl = slice(node_ptr[r], node_ptr[r + 1])
        ref, env = refs[r], envs[r]
        tol = tol_all[: len(env)]
        chk = check_logits(lg_dev[sl].cpu().numpy().astype(np.float64), ref["logits"], tol=tol)
        above.append(chk["row_err"] > 2e-3)
        print(f"  request {r}: {sizes[r]} nodes, ctx {ctxs[r]}: {row_report(chk, env, tol)} "
              f"accepted={int(res.n_accepted[r].item())} (oracle {ref['n_accepted']})", flush=True)
        assert chk["logits_ok"] and chk["argmax_ok"], (r, chk["bad_rows"], chk["max_abs_rel"])
        assert acceptance_ok(am_all[sl], ref["argmax"], toks[r], trees[r], chk["decidable"])
    print(f"  rows above 2e-3: {np.concatenate(above).mean():.3f} of {int(sizes.sum())}; "
          f"batch bound {tol_all[0]:.2e}", flush=True)


class _LazyLayers:
    """Oracle weights of layer l converted from bf16 bits when the forward pass
    reaches it (the whole 4B-like target in fp64 would hold 29 GB at once)."""

    def __init__(self, cfg, seed: int):
        self.cfg, self.seed = cfg, seed

    def __len__(self):
        return self.cfg.n_layers

    def __getitem__(self, layer):
        if not 0 <= layer < self.cfg.n_layers:
            raise IndexError(layer)
        return {k: from_bits(bf16_bits_numpy(v)) for k, v in gen_layer(self.cfg, self.seed, layer, "cpu",
                                                                       "random").items()}

    def __iter__(self):
        return (self[i] for i in range(len(self)))


def test_verify_step_4b_full_depth(cuda):
    """The whole 36-layer 4B-like target, 2048-token context, full LM head, a
    32-node best-first tree whose root's children carry the oracle's own top-4
    tokens (the rest uniform): every row of the logits against the oracle
    under the per-row rule, greedy tokens on decidable rows, acceptance where
    determined, the path following from the pass's own greedy tokens."""
    import tree_verification_pass_amd as tvp
    from synth.configs import gen_embed, gen_final_norm, gen_lm_head
    from tree_verification_pass_amd.model import DeviceModel, Dims

    cfg = CONFIGS["4b"]
    L, s_max, n, seed = cfg.ctx_len, cfg.ctx_len + 64, cfg.n_nodes, 12
    print(f"[full depth] 4b: {cfg.n_layers} layers, ctx {L}, {n} nodes", flush=True)
    kv = [gen_kv_context(cfg, seed, layer, L, s_max) for layer in range(cfg.n_layers)]
    embed = gen_embed(cfg, seed, "cpu")
    fnorm = gen_final_norm(cfg, seed, "cpu", "random")
    lm = gen_lm_head(cfg, seed, "cpu")
    dm = DeviceModel(Dims.of(cfg), embed.to(cuda), fnorm.to(cuda), lm.to(cuda),
                     lambda l: {k: v.to(cuda) for k, v in gen_layer(cfg, seed, l, "cpu", "random").items()},
                     lambda l: (kv[l][0].to(cuda), kv[l][1].to(cuda)), s_max=s_max, max_nodes=n)
    orc = om.OracleModel(om.Dims.of(cfg), _Rows(bf16_bits_numpy(embed)), _LazyLayers(cfg, seed),
                         from_bits(bf16_bits_numpy(fnorm)), from_bits(bf16_bits_numpy(lm)))
    cache = om.KVCache.from_bits([bf16_bits_numpy(k) for k, _ in kv], [bf16_bits_numpy(v) for _, v in kv])
    rng = np.random.default_rng(13)
    parents, rank, _ = best_first_topology(rng, n)
    root = int(rng.integers(cfg.vocab))
    print("  oracle: root's top-4", flush=True)
    lg0, _ = om.forward_tree(orc, cache, L, [root], [-1])
    top = np.argsort(-lg0[0], kind="stable")[:4]
    tokens = rng.integers(0, cfg.vocab, n).astype(np.int32)
    tokens[0] = root
    for i in range(1, n):
        if parents[i] == 0 and rank[i] < 4:
            tokens[i] = int(top[rank[i]])
    print("  oracle forward", flush=True)
    ref = om.verify(orc, cache, L, tokens, parents)
    print("  gpu pass", flush=True)
    res = tvp.verify_step(dm.plan, L, to_i32(tokens), to_i32(parents), commit=False, want_logits=True)
    res2 = tvp.verify_step(dm.plan, L, to_i32(tokens), to_i32(parents), commit=False, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(res.logits, res2.logits)
    g = res.logits.cpu().numpy().astype(np.float64)
    print("  rounding-noise envelope", flush=True)
    env = noise_envelope_rows(orc, cache, L, tokens, parents, ref["logits"], runs=1)
    tol = row_tolerances(env)
    chk = check_logits(g, ref["logits"], tol=tol)
    print(f"  logits {row_report(chk, env, tol)} accepted={int(res.n_accepted.item())} "
          f"(oracle {ref['n_accepted']})", flush=True)
    assert chk["logits_ok"], (chk["bad_rows"], chk["max_abs_rel"])
    assert chk["argmax_ok"], chk["bad_argmax_rows"]
    am = res.argmax.cpu().numpy()
    assert np.array_equal(am, np.argmax(res.logits.cpu().numpy(), axis=1))
    p_own, a_own, b_own = oaccept(am, tokens, parents)
    assert int(res.n_accepted.item()) == a_own and int(res.bonus.item()) == b_own
    assert res.path.cpu().numpy()[: a_own + 1].tolist() == p_own
    assert acceptance_ok(am, ref["argmax"], tokens, parents, chk["decidable"])
    # The in-launch hand-overs (tree attention's split merge, the gate/up
    # GEMM's remaining groups) with two trees alternating on one workspace:
    # a stale read of the other tree's partials, or of another layer's, would
    # change bits; every pass must reproduce its tree's first result exactly.
    rng2 = np.random.default_rng(14)
    parents_b, _, _ = best_first_topology(rng2, n)
    tokens_b = rng2.integers(0, cfg.vocab, n).astype(np.int32)
    tokens_b[0] = root
    first_b = tvp.verify_step(dm.plan, L, to_i32(tokens_b), to_i32(parents_b), commit=False, want_logits=True)
    torch.cuda.synchronize()
    print("  alternating trees, 16 passes", flush=True)
    for it in range(8):
        for tk, pa, want in ((tokens, parents, res.logits), (tokens_b, parents_b, first_b.logits)):
            again = tvp.verify_step(dm.plan, L, to_i32(tk), to_i32(pa), commit=False, want_logits=True)
            torch.cuda.synchronize()
            assert torch.equal(again.logits, want), it
