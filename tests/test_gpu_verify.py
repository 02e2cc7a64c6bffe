"""GPU parity of the whole verification pass (verify_step through the C ABI)
against the CPU oracle: logits within max(2e-3, 1.5 x the row's own rounding-noise
envelope of fp32 evaluations of the same definition -- see
tests/fp32_reference.py), at most 2e-2 per row, greedy tokens equal on decidable rows, acceptance
equal where determined, commit moves exactly the accepted rows, a speculative
loop reproduces the oracle's greedy stream, and a batch gives each request
what the oracle gives that request alone."""

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.accept import accept as oaccept
from synth import best_first_topology, chain_topology
from synth.configs import CONFIGS
from synth.trees import assign_tokens_by_depth
from tests.gpu_util import build_pair, to_i32
from tests.helpers import oracle_topk_fn
from tests.fp32_reference import noise_envelope_rows
from tests.parity import acceptance_ok, check_logits, row_report, row_tolerances

pytestmark = pytest.mark.gpu


def _run(dm, ctx, tokens, parents, commit=False):
    import tree_verification_pass_amd as tvp
    res = tvp.verify_step(dm.plan, ctx, to_i32(tokens), to_i32(parents), commit=commit, want_logits=True)
    torch.cuda.synchronize()
    return res


def _compare(res, ref, tokens, parents, orc, cache, ctx, lg=None):
    g = res.logits.cpu().numpy().astype(np.float64) if lg is None else lg
    env = noise_envelope_rows(orc, cache, ctx, tokens, parents, ref["logits"])
    tol = row_tolerances(env)
    chk = check_logits(g, ref["logits"], tol=tol)
    print(f"  logits {row_report(chk, env, tol)}", flush=True)
    assert chk["logits_ok"], (chk["bad_rows"], chk["max_abs_rel"])
    am = res.argmax.cpu().numpy()
    assert np.array_equal(am, np.argmax(res.logits.cpu().numpy(), axis=1))
    assert chk["argmax_ok"], chk["bad_argmax_rows"]
    assert int(res.status.item()) == 0
    # the result follows from its own greedy tokens, and matches where determined
    p_own, a_own, b_own = oaccept(am, tokens, parents)
    a = int(res.n_accepted.item())
    assert a == a_own and int(res.bonus.item()) == b_own
    assert res.path.cpu().numpy()[: a + 1].tolist() == p_own
    assert acceptance_ok(am, ref["argmax"], tokens, parents, chk["decidable"])
    return chk


@pytest.mark.parametrize("cfg_name", ["tiny", "ragged"])
def test_verify_step_matches_oracle(cuda, cfg_name):
    cfg = CONFIGS[cfg_name]
    print(f"[verify_step] {cfg_name}", flush=True)
    dm, orc, cache = build_pair(cfg, 0, s_max=cfg.ctx_len + 96)
    rng = np.random.default_rng(1)
    for trial in range(3):
        n = cfg.n_nodes if trial == 0 else int(rng.integers(1, 33))
        parents = chain_topology(n) if (cfg.tree == "chain" and trial == 0) else best_first_topology(rng, n)[0]
        tokens = rng.integers(0, cfg.vocab, n).astype(np.int32)
        ref = om.verify(orc, cache, cfg.ctx_len, tokens, parents)
        res = _run(dm, cfg.ctx_len, tokens, parents)
        print(f"  n={n}", flush=True)
        _compare(res, ref, tokens, parents, orc, cache, cfg.ctx_len)
        res2 = _run(dm, cfg.ctx_len, tokens, parents)
        assert torch.equal(res.logits, res2.logits)  # bitwise reproducible


def test_chain_of_greedy_continuation_and_commit(cuda):
    cfg = CONFIGS["tiny"]
    dm, orc, cache = build_pair(cfg, 0, s_max=cfg.ctx_len + 64)
    root = 17
    ar = om.ar_greedy(orc, cache, cfg.ctx_len, root, 8)
    tokens = np.array([root] + ar[:7], dtype=np.int32)
    parents = chain_topology(8)
    ref = om.verify(orc, cache, cfg.ctx_len, tokens, parents)
    assert ref["n_accepted"] == 7
    res = _run(dm, cfg.ctx_len, tokens, parents)
    chk = _compare(res, ref, tokens, parents, orc, cache, cfg.ctx_len)
    if chk["decidable"].all():
        assert int(res.n_accepted.item()) == 7 and int(res.bonus.item()) == ar[7]
    # commit: slots L..L+a hold the accepted nodes' K/V from the pass
    rng = np.random.default_rng(3)
    par2, _, _ = best_first_topology(rng, 20)
    tok2 = rng.integers(0, cfg.vocab, 20).astype(np.int32)
    tok2[0] = root
    tok2[1] = int(np.argmax(ref["logits"][0]))  # node 1 hangs off the root: make it acceptable
    L = cfg.ctx_len
    _run(dm, L, tok2, par2, commit=False)
    snap_k = [l.k_cache.clone() for l in dm.layers]
    snap_v = [l.v_cache.clone() for l in dm.layers]
    res = _run(dm, L, tok2, par2, commit=True)
    a = int(res.n_accepted.item())
    path = res.path.cpu().numpy()[: a + 1]
    for li, layer in enumerate(dm.layers):
        for j, node in enumerate(path):
            assert torch.equal(layer.k_cache[:, L + j], snap_k[li][:, L + node])
            assert torch.equal(layer.v_cache[:, L + j], snap_v[li][:, L + node])
        assert torch.equal(layer.k_cache[:, :L], snap_k[li][:, :L])


def test_speculative_loop_reproduces_greedy_stream(cuda):
    cfg = CONFIGS["tiny"]
    L0 = cfg.ctx_len
    dm, orc, cache = build_pair(cfg, 5, s_max=L0 + 128)
    ref_cache = cache.copy()
    want = 40
    ref_stream = om.ar_greedy(orc, ref_cache, L0, 3, want + 10)
    rng = np.random.default_rng(5)
    ctx, root, stream = L0, 3, []
    while len(stream) < want:
        parents, rank, _ = best_first_topology(rng, 12, max_depth=6)
        tokens = assign_tokens_by_depth(rng, parents, rank, root, cfg.vocab, oracle_topk_fn(orc, cache, ctx),
                                        p_top=0.8)
        ref = om.verify(orc, cache, ctx, tokens, parents)
        res = _run(dm, ctx, tokens, parents, commit=True)
        chk = check_logits(res.logits.cpu().numpy().astype(np.float64), ref["logits"])
        a = int(res.n_accepted.item())
        path = res.path.cpu().numpy()[: a + 1].tolist()
        on_path_decidable = all(chk["decidable"][v] for v in path)
        if not on_path_decidable:
            pytest.skip("a near-tie on the accepted path: the streams may legitimately diverge")
        stream += [int(tokens[v]) for v in path[1:]] + [int(res.bonus.item())]
        ctx = om.commit(cache, ctx, ref["path"], ref["kv_new"])
        assert ref["path"] == path
        root = int(res.bonus.item())
    assert stream[:want] == ref_stream[:want]


def test_ar_decoding_loop_reproduces_greedy_stream(cuda):
    """W12 autoregressive decoding (one node per pass: M = 1, no speculation)
    is the same pass on a one-node tree: its bonus tokens are the oracle's
    greedy stream and its commits keep the cache equal to the oracle's."""
    cfg = CONFIGS["tiny"]
    L0 = cfg.ctx_len
    dm, orc, cache = build_pair(cfg, 7, s_max=L0 + 64)
    want = 24
    ref_stream = om.ar_greedy(orc, cache, L0, 5, want)
    ctx, root, stream = L0, 5, []
    for _ in range(want):
        tokens, parents = np.array([root], np.int32), np.array([-1], np.int32)
        ref = om.verify(orc, cache, ctx, tokens, parents)
        res = _run(dm, ctx, tokens, parents, commit=True)
        chk = check_logits(res.logits.cpu().numpy().astype(np.float64), ref["logits"])
        if not chk["decidable"][0]:
            pytest.skip("a near-tie in the greedy stream: it may legitimately diverge")
        assert int(res.n_accepted.item()) == 0
        root = int(res.bonus.item())
        stream.append(root)
        ctx = om.commit(cache, ctx, ref["path"], ref["kv_new"])
    assert stream == ref_stream


def test_batched_equals_per_request(cuda):
    cfg = CONFIGS["ragged"]
    import tree_verification_pass_amd as tvp
    rng = np.random.default_rng(7)
    # 47 rows in all: the GEMMs take the wide (row-major, more than 32 rows) path
    n_req, s_req = 4, 400
    sizes = [5, 9, 13, 20]
    ctxs = [250, 310, 123, 77]
    dm, orc, cache = build_pair(cfg, 2, s_max=n_req * s_req, max_nodes=64)
    # request r owns slots [r*s_req, (r+1)*s_req): give each its own context
    for layer_i, layer in enumerate(dm.layers):
        for r in range(1, n_req):
            layer.k_cache[:, r * s_req: r * s_req + ctxs[r]] = layer.k_cache[:, : ctxs[r]]
            layer.v_cache[:, r * s_req: r * s_req + ctxs[r]] = layer.v_cache[:, : ctxs[r]]
    trees = [best_first_topology(rng, n)[0] for n in sizes]
    toks = [rng.integers(0, cfg.vocab, n).astype(np.int32) for n in sizes]
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    res = tvp.verify_step_batched(dm.plan, ctxs, node_ptr.tolist(), s_req, to_i32(np.concatenate(toks)),
                                  to_i32(np.concatenate(trees)), commit=False, want_logits=True)
    torch.cuda.synchronize()
    lg = res.logits.cpu().numpy().astype(np.float64)
    for r in range(n_req):
        ref = om.verify(orc, cache, ctxs[r], toks[r], trees[r])
        sl = slice(node_ptr[r], node_ptr[r + 1])
        env = noise_envelope_rows(orc, cache, ctxs[r], toks[r], trees[r], ref["logits"])
        tol = row_tolerances(env)
        chk = check_logits(lg[sl], ref["logits"], tol=tol)
        print(f"  request {r}: {row_report(chk, env, tol)}", flush=True)
        assert chk["logits_ok"] and chk["argmax_ok"], (r, chk["bad_rows"], chk["max_abs_rel"])
        am = res.argmax.cpu().numpy()[sl]
        p_own, a_own, b_own = oaccept(am, toks[r], trees[r])
        assert int(res.n_accepted[r].item()) == a_own and int(res.bonus[r].item()) == b_own
        assert res.path.cpu().numpy()[sl][: a_own + 1].tolist() == p_own
        assert int(res.status[r].item()) == 0
        assert acceptance_ok(am, ref["argmax"], toks[r], trees[r], chk["decidable"])


def test_malformed_tree_and_capacity(cuda):
    import tree_verification_pass_amd as tvp
    cfg = CONFIGS["tiny"]
    dm, _, _ = build_pair(cfg, 0, s_max=cfg.ctx_len + 16)
    res = tvp.verify_step(dm.plan, cfg.ctx_len, to_i32([1, 2, 3]), to_i32([-1, 2, 0]), commit=True)
    torch.cuda.synchronize()
    assert int(res.status.item()) == tvp.TVP_ERR_TREE and int(res.n_accepted.item()) == 0
    with pytest.raises(tvp.TvpError) as e:
        tvp.verify_step(dm.plan, cfg.ctx_len + 10, to_i32(list(range(8))), to_i32(chain_topology(8)))
    assert e.value.status == tvp.TVP_ERR_CAPACITY
    res = tvp.verify_step(dm.plan, cfg.ctx_len, to_i32([1, 99999]), to_i32([-1, 0]), commit=True)
    torch.cuda.synchronize()
    assert int(res.status.item()) == tvp.TVP_ERR_ARG
