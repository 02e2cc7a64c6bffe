"""Pins for the oracle's two-level verification pieces (CPU).

* The 8-bit leading view: over all 65,536 bf16 patterns as one channel (whose
  window base is 1), every in-window pattern reads back with its four low
  mantissa bits cleared and every other pattern exactly; on random weights,
  every in-window value equals the real value truncated toward zero to three
  fraction bits of its binade (computed with floating point, not bit masks),
  so it keeps sign and binade and loses less than 2^-3 of its magnitude.
* The exact tree the second pass checks, on a hand-written case.
* Losslessness of a TLV step: whatever the Q pass gets wrong, the emitted
  tokens (the exact pass's accepted path and bonus) equal step-by-step greedy
  decoding of the exact model; with the greedy continuation drafted, the Q
  pass's matched path carries through and the exact pass accepts at least
  the path and the bonus.
"""

import numpy as np

from oracle import model as om
from oracle import tlv, w12
from oracle.bf16 import from_bits
from synth import best_first_topology, chain_topology, gen_linear_bf16, make_generator
from synth.configs import CONFIGS, LARGE_RECIPE
from synth.weights import bf16_bits_numpy
from tests.helpers import model_bits, oracle_cache


def test_hi8_view_all_patterns():
    allpat = np.random.default_rng(7).permutation(65536).astype(np.uint16)
    t = w12.encode(allpat[None, :])
    assert int(t.base[0]) == 1
    exp = (allpat >> 7) & 0xFF
    inside = (exp >= 1) & (exp <= 16)
    want = np.where(inside, allpat & 0xFFF0, allpat)
    assert np.array_equal(w12.decode_hi8(t)[0], want)


def test_hi8_view_is_truncation_to_three_fraction_bits():
    w = bf16_bits_numpy(gen_linear_bf16(make_generator(5), 64, 777, LARGE_RECIPE))
    t = w12.encode(w)
    q = from_bits(w12.decode_hi8(t))
    x = from_bits(w)
    esc = np.zeros(w.shape, bool)
    rows = np.repeat(np.arange(t.n_out), np.diff(t.esc_ptr.astype(np.int64)))
    esc[rows, t.esc_idx.astype(np.int64)] = True
    assert np.array_equal(w12.decode_hi8(t)[esc], w[esc])  # escapes keep their exact bits
    xi, qi = x[~esc], q[~esc]
    e = np.floor(np.log2(np.abs(xi)))  # binade of every in-window (normal, nonzero) value
    step = np.exp2(e - 3)
    assert np.array_equal(qi, np.sign(xi) * np.floor(np.abs(xi) / step) * step)
    assert np.all(np.abs(qi) <= np.abs(xi)) and np.all(np.abs(xi - qi) < 2.0 ** -3 * np.abs(xi))
    assert np.all(np.floor(np.log2(np.abs(qi))) == e)


def test_exact_tree_by_hand():
    # draft tree: 0 -> 1, 0 -> 2, 2 -> 3, 3 -> 4; Q path 0, 2, 3; bonus 77
    draft_tokens = [10, 11, 12, 13, 14]
    sub_parents = [-1, 0, 0, 1]
    sub_tokens = [77, 80, 81, 82]
    tok, par = tlv.exact_tree([0, 2, 3], draft_tokens, 77, sub_parents, sub_tokens)
    assert tok.tolist() == [10, 12, 13, 77, 80, 81, 82]
    assert par.tolist() == [-1, 0, 1, 2, 3, 3, 4]


def _models(cfg, seed):
    embed, layers, fnorm, lm = model_bits(cfg, seed, "random")
    lin = ("wqkv", "wo", "wgu", "wdown")
    enc = [{k: (w12.encode(v) if k in lin else v) for k, v in layer.items()} for layer in layers]
    lmq = w12.encode(lm)
    dims = om.Dims.of(cfg)
    return (om.OracleModel.from_w12(dims, embed, enc, fnorm, lmq),
            om.OracleModel.from_w12(dims, embed, enc, fnorm, lmq, view="hi8"))


def test_tlv_step_emits_the_greedy_stream():
    cfg = CONFIGS["tiny"]
    exact, q = _models(cfg, 3)
    cache = oracle_cache(cfg, 3, cfg.ctx_len, cfg.ctx_len + 64)
    L, root = cfg.ctx_len, 123
    greedy = om.ar_greedy(exact, cache, L, root, 12)
    rng = np.random.default_rng(4)
    for case in range(3):
        if case == 0:  # the greedy continuation as a chain: the Q path should carry through
            toks = np.array([root] + greedy[:7])
            par = chain_topology(8)
        else:
            par = best_first_topology(rng, 16)[0]
            toks = rng.integers(0, cfg.vocab, 16)
            toks[0] = root

        def redraft(q_path, q_bonus):
            sp = best_first_topology(rng, 32 - len(q_path))[0]
            st = rng.integers(0, cfg.vocab, len(sp))
            st[0] = q_bonus
            return sp, st

        r = tlv.tlv_step(q, exact, cache, L, toks, par, redraft)
        ex = r["exact"]
        assert len(r["tokens"]) == 32
        emitted = [int(r["tokens"][v]) for v in ex["path"][1:]] + [int(ex["bonus"])]
        assert emitted == greedy[: len(emitted)]  # lossless whatever the Q pass did
        if case == 0:
            a_q = len(r["q"]["path"]) - 1
            assert ex["n_accepted"] >= a_q  # the matched path carries through
            if r["q"]["bonus"] == greedy[a_q]:
                assert ex["n_accepted"] >= a_q + 1  # ... and the bonus node too
