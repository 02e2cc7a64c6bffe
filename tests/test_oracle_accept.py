"""Pins for the acceptance walk: exhaustive comparison with root-path enumeration."""

import itertools

import numpy as np
import pytest

from oracle.accept import accept, accept_bruteforce, validate_tree


def all_trees(n):
    """Every recursive tree on n nodes: parents[i] in [0, i)."""
    for tail in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(tail)


@pytest.mark.parametrize("n,alpha", [(1, 2), (2, 3), (3, 3), (4, 3), (5, 2)])
def test_exhaustive_small(n, alpha):
    count = 0
    for parents in all_trees(n):
        for toks in itertools.product(range(alpha), repeat=n - 1):
            tokens = [0] + list(toks)
            for am in itertools.product(range(alpha), repeat=n):
                assert accept(am, tokens, parents) == accept_bruteforce(am, tokens, parents)
                count += 1
    assert count > 0


@pytest.mark.parametrize("n", [6, 7])
def test_every_shape_sampled_assignments(n):
    rng = np.random.default_rng(n)
    shapes = 0
    for parents in all_trees(n):
        shapes += 1
        for _ in range(12):
            tokens = [0] + rng.integers(0, 2, n - 1).tolist()
            am = rng.integers(0, 2, n).tolist()
            assert accept(am, tokens, parents) == accept_bruteforce(am, tokens, parents)
    assert shapes == {6: 120, 7: 720}[n]


def test_random_large_trees():
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(1, 65))
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        tokens = rng.integers(0, 3, n).tolist()
        am = rng.integers(0, 3, n).tolist()
        assert accept(am, tokens, parents) == accept_bruteforce(am, tokens, parents)


def test_chain_special_cases():
    # chain whose drafts all match: every draft accepted, bonus = greedy at the end
    am = [5, 6, 7, 8, 9]
    tokens = [4, 5, 6, 7, 8]
    parents = [-1, 0, 1, 2, 3]
    assert accept(am, tokens, parents) == ([0, 1, 2, 3, 4], 4, 9)
    # first mismatch at node 3: nodes 1, 2 accepted, bonus = greedy after node 2
    tokens2 = [4, 5, 6, 0, 8]
    assert accept(am, tokens2, parents) == ([0, 1, 2], 2, 7)
    # nothing matches: root only, bonus = greedy after the root
    assert accept(am, [4, 0, 0, 0, 0], parents) == ([0], 0, 5)


def test_tie_goes_to_smaller_node_and_bonus_with_children():
    # two accepted depth-1 siblings with the same token: the smaller index wins
    parents = [-1, 0, 0, 1]
    tokens = [0, 3, 3, 9]
    am = [3, 1, 2, 4]
    assert accept(am, tokens, parents) == ([0, 1], 1, 1)
    # bonus is the greedy token at the deepest accepted node even if it has children
    assert accept([3, 8, 2, 4], tokens, parents) == ([0, 1], 1, 8)


@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 0, 2], [-1, -1], []])
def test_malformed_trees_rejected(bad):
    with pytest.raises(ValueError):
        validate_tree(bad)
