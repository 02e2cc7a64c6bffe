"""Seeded draft-tree generators (topology and draft tokens).

The drafter is outside the verification pass; these generators stand in for
it.  A tree is given in topological order: ``parents[0] = -1`` for the root and
``0 <= parents[i] < i`` for every other node.

Topology ("best-first with random parents"): node 0 has score 1 and every node
draws four proposal probabilities ``U(0,1)`` sorted in descending order.  The
next child of node ``v`` (its sibling rank ``c`` = current number of children)
is a candidate while ``c < max_branch`` and ``depth(v) < max_depth``; its
score is ``score(v) * p[v, c]``.  The highest-scoring candidate (ties to the
smaller ``v``) becomes the next node, ``n - 1`` times.

Draft tokens are assigned level by level.  The caller supplies ``topk_fn``,
which returns the target model's top-4 next tokens at every node of the tree
as it stands (nodes below the current level carry token 0, which a tree mask
keeps from influencing shallower nodes).  A child of sibling rank ``c`` takes
its parent's rank-``c`` token with probability ``p_top``, otherwise a uniform
token; a token equal to an already assigned sibling's is replaced by a fresh
uniform draw until it is distinct.
"""

from __future__ import annotations

import heapq
from typing import Callable, List, Sequence, Tuple

import numpy as np


def chain_topology(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def best_first_topology(rng: np.random.Generator, n: int, max_branch: int = 4,
                        max_depth: int = 8) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns ``(parents, sibling_rank, depth)``, each ``int32[n]``."""
    if n < 1:
        raise ValueError("a tree has at least the root")
    parents = np.full(n, -1, dtype=np.int32)
    rank = np.zeros(n, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    score = np.zeros(n, dtype=np.float64)
    probs = np.zeros((n, max_branch), dtype=np.float64)
    nchild = np.zeros(n, dtype=np.int32)

    def draw(v: int) -> None:
        probs[v] = np.sort(rng.random(max_branch))[::-1]

    score[0] = 1.0
    draw(0)
    heap: List[Tuple[float, int]] = []
    if max_depth > 0 and max_branch > 0:
        heapq.heappush(heap, (-score[0] * probs[0, 0], 0))
    for i in range(1, n):
        if not heap:
            raise ValueError(f"cannot grow a {n}-node tree with branching <= {max_branch} "
                             f"and depth <= {max_depth}")
        neg, v = heapq.heappop(heap)
        c = int(nchild[v])
        parents[i] = v
        rank[i] = c
        depth[i] = depth[v] + 1
        score[i] = -neg
        nchild[v] += 1
        draw(i)
        if nchild[v] < max_branch:
            heapq.heappush(heap, (-score[v] * probs[v, nchild[v]], v))
        if depth[i] < max_depth:
            heapq.heappush(heap, (-score[i] * probs[i, 0], i))
    return parents, rank, depth


def depths_of(parents: Sequence[int]) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int32)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def assign_tokens_by_depth(rng: np.random.Generator, parents: np.ndarray, rank: np.ndarray,
                           root_token: int, vocab: int,
                           topk_fn: Callable[[np.ndarray, np.ndarray], np.ndarray],
                           p_top: float = 0.7) -> np.ndarray:
    """Draft tokens for a tree whose topology is fixed (see module docstring)."""
    n = len(parents)
    depth = depths_of(parents)
    tokens = np.zeros(n, dtype=np.int32)
    tokens[0] = int(root_token)
    children: List[List[int]] = [[] for _ in range(n)]
    for i in range(1, n):
        children[parents[i]].append(i)
    maxd = int(depth.max()) if n else 0
    for d in range(maxd):
        level = [v for v in range(n) if depth[v] == d and children[v]]
        if not level:
            continue
        top = np.asarray(topk_fn(tokens.copy(), parents.copy()))
        for v in level:
            taken: List[int] = []
            for ch in children[v]:
                if rng.random() < p_top:
                    t = int(top[v, rank[ch]])
                else:
                    t = int(rng.integers(vocab))
                while t in taken:
                    t = int(rng.integers(vocab))
                tokens[ch] = t
                taken.append(t)
    return tokens


def batch_sizes(rng: np.random.Generator, n_req: int = 24, total: int = 192, start: int = 4,
                cap: int = 16) -> np.ndarray:
    """Per-request node counts sharing one budget: all start at ``start``, then the
    remaining nodes go one at a time to a uniformly chosen request below ``cap``."""
    sizes = np.full(n_req, start, dtype=np.int32)
    left = total - start * n_req
    if left < 0 or total > cap * n_req:
        raise ValueError("budget does not fit the per-request bounds")
    for _ in range(left):
        open_ = np.flatnonzero(sizes < cap)
        sizes[open_[int(rng.integers(len(open_)))]] += 1
    return sizes
