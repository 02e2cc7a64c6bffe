"""Gated DeltaNet layers over a draft tree on the GPU against the oracle
(through the C ABI): the WY-form verify, the path verify and the commit.

Tolerance of an output element (bf16 on the GPU, fp64 in the oracle):
    |gpu - ref| <= 2^-8 |ref| + 2^-14 env
The first term is the final rounding to bf16 (8 significant bits: at most
2^-8 of the value).  The second covers the fp32 arithmetic before it: every
partial sum of either evaluation order is bounded by the oracle's magnitude
envelope ``env`` (the same walk in absolute values), and 2^-14 leaves a
factor 2^10 over one fp32 rounding for the 128-term dot products, the
three-piece state products and the triangular solve of up to 32 nodes.  The
commit's fp32 state is held to 2^-16 of its own envelope (max |S| of the
layer plus |v| |k| of the replayed nodes) per element.
"""

import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from synth import best_first_topology, chain_topology
from synth.gdn import GDN_SHAPES, gen_gdn_inputs
from tests.gpu_util import to_i32

pytestmark = pytest.mark.gpu

REL, ENV = 2.0 ** -8, 2.0 ** -14


@pytest.fixture(scope="module")
def tvp():
    import tree_verification_pass_amd as m
    return m


def _np(inp):
    return [t.double().numpy() for t in (inp.state, inp.q, inp.k, inp.v, inp.g, inp.beta)]


def _dev(inp, dev):
    return [t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state)]


def _check(out, ref, env, what):
    got = out.float().cpu().double().numpy()
    err = np.abs(got - ref)
    tol = REL * np.abs(ref) + ENV * env
    worst = float(np.max(err / tol))
    print(f"{what}: max err/tol {worst:.3f}, max |err| {err.max():.3e}", flush=True)
    assert worst <= 1.0, what


def _tree(kind, n, seed):
    if kind == "chain":
        return chain_topology(n)
    return best_first_topology(np.random.default_rng(seed), n)[0]


@pytest.mark.parametrize("n,kind", [(1, "chain"), (5, "tree"), (17, "tree"), (32, "tree"), (32, "chain"),
                                    (24, "wide")])
def test_gdn_verify_small_matches_oracle(tvp, cuda, n, kind):
    shape = GDN_SHAPES["tiny"]
    inp = gen_gdn_inputs(11, n, n, shape)
    if kind == "wide":  # the root with n - 1 children
        parents = np.array([-1] + [0] * (n - 1), dtype=np.int32)
    else:
        parents = np.asarray(_tree(kind, n, n), dtype=np.int32)
    S, q, k, v, g, b = _np(inp)
    ref = ogdn.tree_outputs(S, q, k, v, g, b, parents)
    env = ogdn.envelope(S, q, k, v, g, b, parents)
    dq, dk, dv, dg, db, ds = _dev(inp, cuda)
    par = to_i32(parents)
    for fn, name in ((tvp.gdn_tree_verify, "wy"), (tvp.gdn_path_verify, "path")):
        out, st = fn(dq, dk, dv, dg, db, ds, par)
        torch.cuda.synchronize()
        assert int(st.item()) == tvp.TVP_OK
        _check(out, ref, env, f"{name} n={n} {kind}")
        again, _ = fn(dq, dk, dv, dg, db, ds, par)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16)), f"{name} not deterministic"


def test_gdn_verify_full_shape_matches_oracle(tvp, cuda):
    """27B-hybrid-like layer: 8 key heads, 40 value heads x 128, a 32-node
    best-first tree (branching <= 4, depth <= 8), every head and node."""
    shape = GDN_SHAPES["27b_hybrid"]
    n = 32
    inp = gen_gdn_inputs(12, 0, n, shape)
    parents = np.asarray(best_first_topology(np.random.default_rng(77), n)[0], dtype=np.int32)
    S, q, k, v, g, b = _np(inp)
    ref = ogdn.tree_outputs(S, q, k, v, g, b, parents)
    env = ogdn.envelope(S, q, k, v, g, b, parents)
    args = _dev(inp, cuda)
    par = to_i32(parents)
    wy, st1 = tvp.gdn_tree_verify(*args, par)
    pa, st2 = tvp.gdn_path_verify(*args, par)
    torch.cuda.synchronize()
    assert int(st1.item()) == tvp.TVP_OK and int(st2.item()) == tvp.TVP_OK
    _check(wy, ref, env, "wy 27b_hybrid")
    _check(pa, ref, env, "path 27b_hybrid")


def test_gdn_malformed_tree_reports_status(tvp, cuda):
    shape = GDN_SHAPES["tiny"]
    inp = gen_gdn_inputs(13, 0, 6, shape)
    args = _dev(inp, cuda)
    for bad in ([-1, 0, 5, 1, 2, 3], [0, 0, 1, 2, 3, 4], [-1, 0, 1, -1, 2, 3]):
        for fn in (tvp.gdn_tree_verify, tvp.gdn_path_verify):
            _, st = fn(*args, to_i32(bad))
            torch.cuda.synchronize()
            assert int(st.item()) == tvp.TVP_ERR_TREE


def test_gdn_rejects_bad_shapes(tvp, cuda):
    shape = GDN_SHAPES["tiny"]
    inp = gen_gdn_inputs(14, 0, 4, shape)
    q, k, v, g, b, s = _dev(inp, cuda)
    par = to_i32([-1, 0, 1, 2])
    with pytest.raises(tvp.TvpError):
        tvp.gdn_tree_verify(q[:, :, :64].contiguous(), k[:, :, :64].contiguous(), v, g, b,
                            s[:, :, :64].contiguous(), par)
    with pytest.raises(tvp.TvpError):  # 3 value heads over 2 key heads
        tvp.gdn_path_verify(q, k, v[:, :3].contiguous(), g[:, :3].contiguous(), b[:, :3].contiguous(),
                            s[:3].contiguous(), par)


def _stack(layers, n, shape, seed):
    inps = [gen_gdn_inputs(seed, l, n, shape) for l in range(layers)]
    st = torch.stack([i.state for i in inps])
    k = torch.stack([i.k for i in inps])
    v = torch.stack([i.v for i in inps])
    g = torch.stack([i.g for i in inps])
    b = torch.stack([i.beta for i in inps])
    return inps, st, k, v, g, b


def test_gdn_commit_matches_oracle(tvp, cuda):
    shape = GDN_SHAPES["tiny"]
    L, n = 3, 20
    parents = np.asarray(best_first_topology(np.random.default_rng(5), n)[0], dtype=np.int32)
    leaf = n - 1
    path = ogdn.root_path(parents, leaf)
    inps, st, k, v, g, b = _stack(L, n, shape, 21)
    dst = st.to(cuda).contiguous()
    pbuf = np.full(n, -1, dtype=np.int32)
    pbuf[:len(path)] = path
    na = to_i32([len(path) - 1])
    ok = to_i32([tvp.TVP_OK])
    tvp.gdn_commit(dst, k.to(cuda), v.to(cuda), g.to(cuda), b.to(cuda), to_i32(pbuf), na, ok)
    torch.cuda.synchronize()
    got = dst.cpu().double().numpy()
    for l in range(L):
        S, q, kk, vv, gg, bb = _np(inps[l])
        ref = ogdn.commit(S, kk, vv, gg, bb, path)
        scale = np.abs(S).max() + sum(np.abs(vv[j]).max() * np.abs(kk[j]).max() for j in path)
        err = np.abs(got[l] - ref).max()
        print(f"commit layer {l}: max |err| {err:.3e}, bound {2.0 ** -16 * scale:.3e}", flush=True)
        assert err <= 2.0 ** -16 * scale


def test_gdn_commit_skips_on_bad_status_or_length(tvp, cuda):
    shape = GDN_SHAPES["tiny"]
    L, n = 2, 8
    _, st, k, v, g, b = _stack(L, n, shape, 22)
    args = [t.to(cuda).contiguous() for t in (k, v, g, b)]
    path = to_i32([0, 1, 2, 3, -1, -1, -1, -1])
    for na, status in ((3, 3), (8, 0), (-1, 0)):  # TVP_ERR_TREE; n_accepted out of range (twice)
        dst = st.to(cuda).contiguous()
        tvp.gdn_commit(dst, *args, path, to_i32([na]), to_i32([status]))
        torch.cuda.synchronize()
        assert torch.equal(dst.cpu(), st)
    dst = st.to(cuda).contiguous()  # a path entry out of range
    tvp.gdn_commit(dst, *args, to_i32([0, 9, 2, 3, -1, -1, -1, -1]), to_i32([2]), to_i32([0]))
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), st)


def test_gdn_commit_then_verify_equals_longer_tree(tvp, cuda):
    """Commit a path of one tree on the GPU, verify a second tree from the new
    state; the oracle's outputs for the tree holding the path as a chain with
    the second tree below it are the reference."""
    shape = GDN_SHAPES["tiny"]
    n1, n2 = 12, 9
    p1 = np.asarray(best_first_topology(np.random.default_rng(31), n1)[0], dtype=np.int32)
    path = ogdn.root_path(p1, n1 - 1)
    a = gen_gdn_inputs(41, 0, n1, shape)
    bnext = gen_gdn_inputs(42, 0, n2, shape)
    p2 = np.asarray(best_first_topology(np.random.default_rng(32), n2)[0], dtype=np.int32)
    dst = a.state.unsqueeze(0).to(cuda).contiguous()
    pbuf = np.full(n1, -1, dtype=np.int32)
    pbuf[:len(path)] = path
    tvp.gdn_commit(dst, *(t.unsqueeze(0).to(cuda).contiguous() for t in (a.k, a.v, a.g, a.beta)), to_i32(pbuf),
                   to_i32([len(path) - 1]), to_i32([tvp.TVP_OK]))
    out, st = tvp.gdn_tree_verify(*(t.to(cuda).contiguous() for t in (bnext.q, bnext.k, bnext.v, bnext.g, bnext.beta)),
                                  dst[0], to_i32(p2))
    torch.cuda.synchronize()
    assert int(st.item()) == tvp.TVP_OK
    sel = np.array(path)
    L = len(path)
    par = np.array(list(chain_topology(L)) + [L - 1 if p < 0 else L + p for p in p2], dtype=np.int32)
    A, B = _np(a), _np(bnext)
    cat = [np.concatenate([A[i][sel], B[i]]) for i in range(1, 6)]
    ref = ogdn.tree_outputs(A[0], *cat, par)[L:]
    env = ogdn.envelope(A[0], *cat, par)[L:]
    _check(out, ref, env, "commit then verify")
