"""Gated DeltaNet layers of a hybrid target over a draft tree: the outputs of
every node and the state after the accepted path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: SpecPilot summary (onedev.kr), section 무엇과 다른가 -- for hybrid
targets whose recurrent layers are Gated DeltaNet, verification recomputes the
recurrent state along each root path instead of keeping a copy per node, and
after acceptance the accepted path is replayed into every recurrent layer.

The page names the layer but does not define it; the recurrence is the gated
delta rule as published with Gated DeltaNet (Yang, Kautz and Hatamizadeh,
"Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025), read
with these conventions:

* per value head h the state S is a ``dv x dk`` matrix (rows: value
  dimensions, columns: key dimensions);
* a token with key k, value v, log decay g (alpha = exp(g), g <= 0) and write
  strength beta updates it as
  ``S <- alpha * S (I - beta k k^T) + beta v k^T``
  ``   = alpha * S + beta * (v - alpha * S k) k^T``;
* its output is ``o = S q`` with the state after its own update;
* q and k come from key head ``h // (hv // hk)`` (several value heads share a
  key head); q, k and v are given after whatever projection, convolution and
  normalisation the layer applies before the recurrence.

Over a draft tree (nodes in topological order, ``parents[0] = -1``) every node
is a new token: node i's state is the committed state with the updates of the
root-to-i path applied in root-first order.  fp64 throughout.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .accept import validate_tree


def root_path(parents: Sequence[int], i: int) -> List[int]:
    """Nodes from the root to ``i`` (root first)."""
    path = [int(i)]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    path.reverse()
    return path


def update(S: np.ndarray, k: np.ndarray, v: np.ndarray, g: float, beta: float) -> np.ndarray:
    """One gated delta-rule update of a ``dv x dk`` state (returns a new array)."""
    a = np.exp(np.float64(g))
    return a * S + np.float64(beta) * np.outer(v - a * (S @ k), k)


def _check(state, q, k, v, g, beta):
    hv, dv, dk = state.shape
    n, hk, dk2 = k.shape
    if dk2 != dk or q.shape != k.shape or v.shape != (n, hv, dv) or g.shape != (n, hv) or beta.shape != (n, hv):
        raise ValueError("inconsistent shapes")
    if hk < 1 or hv % hk:
        raise ValueError("value heads must be a multiple of key heads")
    return n, hk, hv, dk, dv


def tree_outputs(state, q, k, v, g, beta, parents) -> np.ndarray:
    """Outputs ``o[i, h] = S_i q_i`` of every node, ``[n, hv, dv]`` fp64.

    ``state`` ``[hv, dv, dk]`` is the committed state; ``q, k`` ``[n, hk, dk]``,
    ``v`` ``[n, hv, dv]``, ``g, beta`` ``[n, hv]``.  Each node's state is
    recomputed from the committed one along its own root path."""
    state, q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (state, q, k, v, g, beta))
    n, hk, hv, dk, dv = _check(state, q, k, v, g, beta)
    validate_tree(parents)
    grp = hv // hk
    out = np.zeros((n, hv, dv))
    for i in range(n):
        path = root_path(parents, i)
        for h in range(hv):
            kh = h // grp
            S = state[h]
            for j in path:
                S = update(S, k[j, kh], v[j, h], g[j, h], beta[j, h])
            out[i, h] = S @ q[i, kh]
    return out


def commit(state, k, v, g, beta, path: Sequence[int]) -> np.ndarray:
    """The state after the accepted path (node indices, root first) is
    replayed into the committed state: ``[hv, dv, dk]`` fp64."""
    state, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (state, k, v, g, beta))
    hv = state.shape[0]
    hk = k.shape[1]
    grp = hv // hk
    out = state.copy()
    for h in range(hv):
        S = state[h]
        for j in path:
            S = update(S, k[j, h // grp], v[j, h], g[j, h], beta[j, h])
        out[h] = S
    return out


def envelope(state, q, k, v, g, beta, parents) -> np.ndarray:
    """Magnitude envelope of every output, ``[n, hv, dv]``: the same walk with
    |S|, |k|, |q|, |v| and the delta's two parts added in absolute value.  It
    bounds every partial sum a reordered fp32 evaluation of the output forms,
    so it scales the arithmetic part of a tolerance."""
    state, q, k, v, beta = (np.abs(np.asarray(x, dtype=np.float64)) for x in (state, q, k, v, beta))
    g = np.asarray(g, dtype=np.float64)
    n, hk, hv, dk, dv = _check(state, q, k, v, g, beta)
    grp = hv // hk
    out = np.zeros((n, hv, dv))
    for i in range(n):
        path = root_path(parents, i)
        for h in range(hv):
            kh = h // grp
            E = state[h]
            for j in path:
                a = np.exp(g[j, h])
                E = a * E + beta[j, h] * np.outer(v[j, h] + a * (E @ k[j, kh]), k[j, kh])
            out[i, h] = E @ q[i, kh]
    return out
