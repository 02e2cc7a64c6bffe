"""Host checks of the synthetic input generators (no method arithmetic here)."""

import numpy as np
import torch

from synth import LinearRecipe, batch_sizes, best_first_topology, chain_topology, gen_linear_bf16, make_generator
from synth.trees import assign_tokens_by_depth, depths_of


def test_best_first_topology_properties():
    for seed in range(20):
        rng = np.random.default_rng(seed)
        parents, rank, depth = best_first_topology(rng, 32)
        assert parents[0] == -1
        assert all(0 <= parents[i] < i for i in range(1, 32))
        assert depth.max() <= 8
        counts = np.bincount(parents[1:], minlength=32)
        assert counts.max() <= 4
        for i in range(1, 32):
            sib = [j for j in range(1, i) if parents[j] == parents[i]]
            assert rank[i] == len(sib)
        assert np.array_equal(depth, depths_of(parents))
    p1 = best_first_topology(np.random.default_rng(5), 32)[0]
    p2 = best_first_topology(np.random.default_rng(5), 32)[0]
    assert np.array_equal(p1, p2)


def test_tokens_follow_topk_and_siblings_distinct():
    rng = np.random.default_rng(1)
    parents, rank, _ = best_first_topology(rng, 32)
    calls = []

    def topk(tokens, par):
        calls.append(1)
        n = len(tokens)
        # a deterministic stand-in: top-4 of node v are 100v+1..100v+4
        return np.array([[100 * v + c + 1 for c in range(4)] for v in range(n)])

    toks = assign_tokens_by_depth(rng, parents, rank, 7, 5000, topk, p_top=1.0)
    assert toks[0] == 7
    for i in range(1, 32):
        assert toks[i] == 100 * parents[i] + rank[i] + 1
    assert len(calls) <= 8
    toks = assign_tokens_by_depth(np.random.default_rng(2), parents, rank, 7, 3, topk, p_top=0.0)
    for v in range(32):
        ch = [toks[i] for i in range(1, 32) if parents[i] == v]
        assert len(set(ch)) == len(ch)


def test_batch_sizes():
    s = batch_sizes(np.random.default_rng(0))
    assert s.sum() == 192 and s.min() >= 4 and s.max() <= 16 and len(s) == 24


def test_linear_recipe_counts():
    g = make_generator(3)
    w = gen_linear_bf16(g, 10, 1000, LinearRecipe(sigma=0.02, zero_frac=0.01, outlier_frac=0.002,
                                                   outlier_mult=300.0))
    x = w.float()
    assert torch.all((x == 0).sum(dim=1) >= 10)
    assert torch.all((x.abs() > 1.0).sum(dim=1) >= 1)
    assert chain_topology(4).tolist() == [-1, 0, 1, 2]
