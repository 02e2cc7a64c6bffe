"""Pins for the oracle's certified INT8 LM head (CPU).

* The certificate, by brute force: on many small random heads -- with exact
  zeros, rare large outliers, duplicated rows (exact ties) and near-ties --
  the argmax over the certified candidates equals the argmax of the whole
  exact row (ties to the smallest id), and every exact logit lies within the
  Cauchy-Schwarz bound of its approximation.
* The encoding: the n largest magnitudes of each row are the escapes, the
  int8 values lie in [-127, 127] and each stands within half a scale step of
  its weight, and the stored residual norm is not below the exact one.
* The bound is what certifies: on heads whose rows are near-copies of one
  another (exact logits closer than the quantization error), the certified
  set still yields the exact argmax, and the same filter with the bound
  shrunk a hundredfold loses it on some rows.
* On the large-recipe weights the filter leaves only a handful of the
  vocabulary per row; with a per-row scale set by the outliers it would not.
"""

import numpy as np
from oracle import lmhead_i8 as oh
from oracle.bf16 import from_bits, round_bf16, to_bits
from synth import LinearRecipe, gen_linear_bf16, make_generator
from synth.configs import LARGE_RECIPE
from synth.weights import bf16_bits_numpy


def _case(seed, V, k):
    rec = LinearRecipe(sigma=None, sigma_lo=0.005, sigma_hi=0.05, zero_frac=0.02, outlier_frac=0.004,
                       outlier_mult=1000.0)
    w = bf16_bits_numpy(gen_linear_bf16(make_generator(seed), V, k, rec))
    rng = np.random.default_rng(seed)
    dup = rng.choice(V, size=V // 8, replace=False)
    w[dup[1:]] = w[dup[0]]  # exact ties between rows
    f = round_bf16(rng.standard_normal((6, k)))
    f[0] = 0.0  # all logits equal: the smallest id wins
    return w, f


def _exact_argmax(f, w_bits):
    return np.argmax(np.asarray(f, np.float64) @ from_bits(w_bits).T, axis=1)


def test_certificate_brute_force():
    for seed in range(40):
        V, k = (64, 40) if seed % 2 else (257, 96)
        w, f = _case(seed, V, k)
        head = oh.encode(w)
        exact = np.asarray(f, np.float64) @ from_bits(w).T
        a = oh.approx_logits(f, head)
        b = np.linalg.norm(f, axis=1)[:, None] * head.r.astype(np.float64)[None, :]
        assert np.all(np.abs(exact - a) <= b * (1 + 1e-12) + 1e-300)
        assert np.array_equal(oh.argmax(f, head, w), _exact_argmax(f, w))


def test_encoding():
    w, _ = _case(3, 200, 130)
    head = oh.encode(w)
    x = from_bits(w)
    mag = np.abs(x)
    for v in range(200):
        esc = set(head.esc_col[v].tolist())
        order = sorted(range(130), key=lambda c: (-mag[v, c], c))
        assert esc == set(order[:8])
        rest = [c for c in range(130) if c not in esc]
        qv = head.q[v, rest].astype(np.float64)
        assert np.all(np.abs(qv) <= 127)
        s = float(head.scale[v])
        assert np.all(np.abs(x[v, rest] - s * qv) <= 0.5 * s + 127 * s * 2.0 ** -22)  # rounding of s and w / s
    err = x - head.scale.astype(np.float64)[:, None] * head.dequant()
    assert np.all(head.r.astype(np.float64) >= np.sqrt(np.sum(err * err, axis=1)))


def test_shrunken_bound_loses_the_argmax():
    missed = 0
    for seed in range(20):
        rng = np.random.default_rng(100 + seed)
        base = 0.02 * rng.standard_normal(80)
        w = np.stack([round_bf16(base + 2e-5 * rng.standard_normal(80)) for _ in range(64)])
        wb = to_bits(w)
        f = round_bf16(rng.standard_normal((6, 80)))
        head = oh.encode(wb)
        assert np.array_equal(oh.argmax(f, head, wb), _exact_argmax(f, wb))  # certified with the true bound
        head.r = (head.r / 100).astype(np.float32)
        missed += int(np.sum(oh.argmax(f, head, wb) != _exact_argmax(f, wb)))
    assert missed > 0


def test_filter_is_selective_on_large_recipe_weights():
    w = bf16_bits_numpy(gen_linear_bf16(make_generator(7), 4096, 5120, LARGE_RECIPE))
    f = round_bf16(np.random.default_rng(8).standard_normal((4, 5120)))
    cand = oh.candidates(f, oh.encode(w))
    assert cand.sum(axis=1).max() <= 8
    # a per-row scale set by the outliers (no escapes) keeps far more of the vocabulary
    wide = oh.candidates(f, oh.encode(w, n_esc=0))
    assert wide.sum(axis=1).min() > 20 * cand.sum(axis=1).max()
