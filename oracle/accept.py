"""Greedy acceptance over a draft tree: the matched path and the bonus token.

Source: SpecPilot summary (onedev.kr), section 무엇과 다른가 -- verification
yields the path of the draft tree that the target agrees with, plus one bonus
token taken from the target at the path's end.

Tree encoding (a reading): nodes in topological order, ``parents[0] = -1``
(the root, which is the last committed token) and ``0 <= parents[i] < i``.
``argmax[v]`` is the target's greedy next token after the root-to-``v``
prefix.  A node is accepted when its parent is accepted and its draft token
equals the parent's greedy token; the root is always accepted.  The result is
the deepest accepted node (the smallest index among equally deep ones), the
root-to-it path, the number of accepted draft tokens (its depth) and the
bonus token ``argmax`` at that node.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def validate_tree(parents: Sequence[int]) -> None:
    p = list(parents)
    if len(p) == 0:
        raise ValueError("empty tree")
    if p[0] != -1:
        raise ValueError("parents[0] must be -1")
    for i in range(1, len(p)):
        if not (0 <= p[i] < i):
            raise ValueError(f"parents[{i}] = {p[i]} is not in [0, {i})")


def depths(parents: Sequence[int]) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def accept(argmax: Sequence[int], tokens: Sequence[int], parents: Sequence[int]
           ) -> Tuple[List[int], int, int]:
    """Acceptance walk in node order: returns ``(path, n_accepted, bonus)``."""
    validate_tree(parents)
    n = len(parents)
    ok = [False] * n
    dep = [0] * n
    ok[0] = True
    best = 0
    for i in range(1, n):
        p = parents[i]
        dep[i] = dep[p] + 1
        ok[i] = ok[p] and int(tokens[i]) == int(argmax[p])
        if ok[i] and dep[i] > dep[best]:
            best = i
    path = [best]
    while path[-1] != 0:
        path.append(parents[path[-1]])
    path.reverse()
    return path, len(path) - 1, int(argmax[best])


def accept_bruteforce(argmax: Sequence[int], tokens: Sequence[int], parents: Sequence[int]
                      ) -> Tuple[List[int], int, int]:
    """Definition by enumeration: every root path is checked on its own, the
    longest fully matching one wins (smallest end node on ties)."""
    validate_tree(parents)
    best_path: List[int] = [0]
    for v in range(len(parents)):
        path = [v]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path.reverse()
        if all(int(tokens[path[j + 1]]) == int(argmax[path[j]]) for j in range(len(path) - 1)):
            if len(path) > len(best_path):
                best_path = path
    return best_path, len(best_path) - 1, int(argmax[best_path[-1]])
