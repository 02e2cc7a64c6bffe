"""Pins for the oracle's Gated DeltaNet tree outputs and commit (CPU).

* The update's defining properties: with alpha = beta = 1 and a unit key the
  state maps the key to the value exactly; a direction orthogonal to the key
  only decays; the factored form ``alpha S (I - beta k k^T) + beta v k^T``
  (written as explicit matrices) equals the oracle's update.
* A hand-computed scalar tree (root, child, sibling), numbers worked out in
  the docstring.
* No writes (beta = 0): every output is the committed state decayed by the
  product of its root path's alphas.
* Tree structure: a node's output equals the last output of the chain made of
  its root path; changing a node outside that path leaves it alone, changing
  one on it does not.
* Shared key heads: repeating each key head over its value heads gives the
  same outputs with one key head per value head.
* The WY form the GPU uses (solve of the unit lower-triangular ancestor
  system, by numpy.linalg.solve) reproduces every output.
* Commit: replaying a node's root path gives a state whose product with that
  node's query is its output; committing a path and then verifying a subtree
  equals verifying the tree that contains both.
* The magnitude envelope bounds every output.
"""

import numpy as np
import pytest

from oracle import gdn
from synth import best_first_topology, chain_topology
from synth.gdn import GDN_SHAPES, gen_gdn_inputs


def _rand(rng, n, hk, hv, dk, dv):
    k = rng.standard_normal((n, hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((n, hk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((n, hv, dv))
    g = np.log(rng.uniform(0.8, 1.0, (n, hv)))
    beta = rng.uniform(0.05, 0.95, (n, hv))
    state = 0.3 * rng.standard_normal((hv, dv, dk))
    return state, q, k, v, g, beta


def test_update_writes_value_at_unit_key():
    rng = np.random.default_rng(1)
    S = rng.standard_normal((5, 7))
    k = rng.standard_normal(7)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(5)
    assert np.allclose(gdn.update(S, k, v, 0.0, 1.0) @ k, v, atol=1e-12)


def test_update_only_decays_orthogonal_directions():
    rng = np.random.default_rng(2)
    S = rng.standard_normal((6, 9))
    k = rng.standard_normal(9)
    x = rng.standard_normal(9)
    x -= (x @ k) / (k @ k) * k
    v = rng.standard_normal(6)
    g = np.log(0.7)
    assert np.allclose(gdn.update(S, k, v, g, 0.4) @ x, 0.7 * (S @ x), atol=1e-12)


def test_update_equals_factored_form():
    rng = np.random.default_rng(3)
    S = rng.standard_normal((4, 6))
    k = rng.standard_normal(6)
    v = rng.standard_normal(4)
    alpha, beta = 0.85, 0.3
    want = alpha * S @ (np.eye(6) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    assert np.allclose(gdn.update(S, k, v, np.log(alpha), beta), want, atol=1e-12)


def test_hand_computed_scalar_tree():
    """dk = dv = 1, one head; committed state 2; nodes (parent, k, v, alpha,
    beta, q):  0: (-1, 0.5, 3, 0.5, 0.25, 2),  1: (0, 1, -1, 1, 0.5, 4),
    2: (0, -1, 1, 0.25, 1, 1).
    Node 0: 0.5*2 + 0.25*(3 - 0.5*2*0.5)*0.5 = 1.3125, output 2.625.
    Node 1: 1.3125 + 0.5*(-1 - 1.3125)*1 = 0.15625, output 0.625.
    Node 2: 0.25*1.3125 + 1*(1 - 0.25*1.3125*(-1))*(-1) = -1, output -1."""
    parents = [-1, 0, 0]
    k = np.array([0.5, 1.0, -1.0]).reshape(3, 1, 1)
    q = np.array([2.0, 4.0, 1.0]).reshape(3, 1, 1)
    v = np.array([3.0, -1.0, 1.0]).reshape(3, 1, 1)
    g = np.log(np.array([0.5, 1.0, 0.25])).reshape(3, 1)
    beta = np.array([0.25, 0.5, 1.0]).reshape(3, 1)
    state = np.array([[[2.0]]])
    out = gdn.tree_outputs(state, q, k, v, g, beta, parents)
    assert np.allclose(out[:, 0, 0], [2.625, 0.625, -1.0], atol=1e-14)
    assert np.allclose(gdn.commit(state, k, v, g, beta, [0, 1])[0, 0, 0], 0.15625, atol=1e-14)


def test_no_writes_is_decay_along_the_root_path():
    rng = np.random.default_rng(4)
    parents = best_first_topology(rng, 20)[0]
    state, q, k, v, g, beta = _rand(rng, 20, 2, 4, 8, 6)
    beta[:] = 0.0
    out = gdn.tree_outputs(state, q, k, v, g, beta, parents)
    for i in range(20):
        j, logd = i, 0.0
        while j >= 0:  # the decay of every ancestor and of the node itself
            logd += g[j]
            j = parents[j]
        for h in range(4):
            assert np.allclose(out[i, h], np.exp(logd[h]) * state[h] @ q[i, h // 2], atol=1e-12)


def test_output_depends_on_the_root_path_only():
    rng = np.random.default_rng(5)
    n = 24
    parents = best_first_topology(rng, n)[0]
    state, q, k, v, g, beta = _rand(rng, n, 2, 4, 8, 8)
    out = gdn.tree_outputs(state, q, k, v, g, beta, parents)
    for i in (5, 13, n - 1):
        path = gdn.root_path(parents, i)
        sel = np.array(path)
        chain = gdn.tree_outputs(state, q[sel], k[sel], v[sel], g[sel], beta[sel], chain_topology(len(path)))
        assert np.allclose(chain[-1], out[i], atol=1e-12)
        off = [j for j in range(n) if j not in path]
        v2 = v.copy()
        v2[off] += 1.0
        assert np.allclose(gdn.tree_outputs(state, q, k, v2, g, beta, parents)[i], out[i], atol=1e-12)
        v3 = v.copy()
        v3[path[0]] += 1.0
        assert not np.allclose(gdn.tree_outputs(state, q, k, v3, g, beta, parents)[i], out[i], atol=1e-6)


def test_key_heads_shared_by_value_heads():
    rng = np.random.default_rng(6)
    parents = best_first_topology(rng, 10)[0]
    state, q, k, v, g, beta = _rand(rng, 10, 2, 6, 8, 4)
    out = gdn.tree_outputs(state, q, k, v, g, beta, parents)
    rep = np.repeat(np.arange(2), 3)  # value head h reads key head h // 3
    out2 = gdn.tree_outputs(state, q[:, rep], k[:, rep], v, g, beta, parents)
    assert np.allclose(out, out2, atol=1e-13)


def _wy_outputs(state, q, k, v, g, beta, parents):
    """All outputs from one linear solve per head: with G_i the sum of g over
    node i's root path (node included) and u_i = beta_i (v_i - alpha_i S_{p(i)} k_i)
    the write of node i,
      (I + A) U = beta (V - e^G (K S0^T)),  A_ij = beta_i e^(G_i - G_j) k_i.k_j  (j a strict ancestor of i)
      O = e^G (Q S0^T) + (M o e^(G_i - G_j) o Q K^T) U  (M: j an ancestor of i or i itself)."""
    n, hk, _ = k.shape
    hv = state.shape[0]
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in gdn.root_path(parents, i):
            anc[i, j] = True
    G = np.array([[g[gdn.root_path(parents, i), h].sum() for h in range(hv)] for i in range(n)])
    out = np.zeros((n, hv, state.shape[1]))
    for h in range(hv):
        kh = h // (hv // hk)
        K, Q, V, S0 = k[:, kh], q[:, kh], v[:, h], state[h]
        E = np.exp(G[:, h][:, None] - G[:, h][None, :])
        strict = anc & ~np.eye(n, dtype=bool)
        A = np.where(strict, beta[:, h][:, None] * E * (K @ K.T), 0.0)
        B = beta[:, h][:, None] * (V - np.exp(G[:, h])[:, None] * (K @ S0.T))
        U = np.linalg.solve(np.eye(n) + A, B)
        out[:, h] = np.exp(G[:, h])[:, None] * (Q @ S0.T) + np.where(anc, E * (Q @ K.T), 0.0) @ U
    return out


def test_wy_form_reproduces_every_output():
    rng = np.random.default_rng(7)
    for n in (1, 7, 32):
        parents = best_first_topology(rng, n)[0]
        state, q, k, v, g, beta = _rand(rng, n, 2, 4, 16, 8)
        want = gdn.tree_outputs(state, q, k, v, g, beta, parents)
        assert np.allclose(_wy_outputs(state, q, k, v, g, beta, parents), want, atol=1e-10)


def test_commit_matches_outputs_and_composes():
    rng = np.random.default_rng(8)
    n = 16
    parents = best_first_topology(rng, n)[0]
    state, q, k, v, g, beta = _rand(rng, n, 1, 2, 8, 8)
    out = gdn.tree_outputs(state, q, k, v, g, beta, parents)
    i = n - 1
    path = gdn.root_path(parents, i)
    S = gdn.commit(state, k, v, g, beta, path)
    for h in range(2):
        assert np.allclose(S[h] @ q[i, 0], out[i, h], atol=1e-12)
    # commit a path of a first tree, then verify a second tree from the new
    # state: the same as one tree holding the path as a chain with the second
    # tree hung below its end
    m = 6
    p2 = best_first_topology(rng, m)[0]
    s2, q2, k2, v2, g2, b2 = _rand(rng, m, 1, 2, 8, 8)
    after = gdn.tree_outputs(S, q2, k2, v2, g2, b2, p2)
    L = len(path)
    sel = np.array(path)
    par = list(chain_topology(L)) + [L - 1 if p < 0 else L + p for p in p2]
    cat = lambda a, b: np.concatenate([a[sel], b])  # noqa: E731
    both = gdn.tree_outputs(state, cat(q, q2), cat(k, k2), cat(v, v2), cat(g, g2), cat(beta, b2), par)
    assert np.allclose(both[L:], after, atol=1e-12)


def test_envelope_bounds_outputs():
    inp = gen_gdn_inputs(3, 0, 12, GDN_SHAPES["tiny"])
    parents = best_first_topology(np.random.default_rng(9), 12)[0]
    args = [t.double().numpy() for t in (inp.state, inp.q, inp.k, inp.v, inp.g, inp.beta)]
    out = gdn.tree_outputs(*args, parents)
    env = gdn.envelope(*args, parents)
    assert np.all(np.abs(out) <= env * (1 + 1e-12))


def test_rejects_bad_tree_and_shapes():
    rng = np.random.default_rng(10)
    state, q, k, v, g, beta = _rand(rng, 3, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        gdn.tree_outputs(state, q, k, v, g, beta, [-1, 1, 0])
    with pytest.raises(ValueError):
        gdn.tree_outputs(state[:, :, :3], q, k, v, g, beta, [-1, 0, 0])
