"""Pins for the oracle's W12 encoder/decoder.

* lossless: bit-exact round trip over all 65,536 bf16 patterns (NaN payloads
  included), as one channel and as a 256x256 matrix, and on random weights;
* the hand-worked two-channel fixture in tests/golden (bytes, bases, escapes);
* the window rule checked against an exhaustive search over every base;
* size: bits/weight of Gaussian weights against the closed form from the
  normal distribution's binade probabilities.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import erf

from oracle import w12
from synth import LinearRecipe, gen_linear_bf16, make_generator
from synth.weights import bf16_bits_numpy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w12_handworked.json")


def _h(xs):
    return np.array([int(x, 16) for x in xs])


def test_handworked_fixture():
    g = json.load(open(GOLDEN))
    w = np.array([_h(r) for r in g["weights"]], dtype=np.uint16)
    t = w12.encode(w)
    assert t.base.tolist() == g["base"]
    assert np.array_equal(t.hi, np.array([_h(r) for r in g["hi"]], dtype=np.uint8))
    assert np.array_equal(t.lo, np.array([_h(r) for r in g["lo"]], dtype=np.uint8))
    assert t.esc_ptr.tolist() == g["esc_ptr"]
    assert t.esc_idx.tolist() == g["esc_idx"]
    assert t.esc_val.tolist() == _h(g["esc_val"]).tolist()
    assert np.array_equal(w12.decode(t), w)


def test_all_patterns_one_channel():
    pats = np.random.default_rng(7).permutation(65536).astype(np.uint16)[None, :]
    t = w12.encode(pats)
    # every exponent holds 256 patterns, so every window ties at 16*256 = 4096
    # in-window patterns: the smallest base (1) wins and 65536 - 4096 escape.
    assert int(t.base[0]) == 1
    assert t.n_esc == 61440
    assert np.array_equal(w12.decode(t), pats)
    # escape indices ascend within the channel
    assert np.all(np.diff(t.esc_idx.astype(np.int64)) > 0)


def test_all_patterns_matrix():
    pats = np.random.default_rng(8).permutation(65536).astype(np.uint16).reshape(256, 256)
    t = w12.encode(pats)
    assert np.array_equal(w12.decode(t), pats)
    assert t.esc_ptr[-1] == t.esc_idx.size


@pytest.mark.parametrize("n,k", [(5, 1), (3, 7), (17, 64), (33, 1000)])
def test_random_roundtrip_and_window_rule(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    # a mix of scales per channel plus specials
    sig = 10.0 ** rng.uniform(-8, 3, size=(n, 1))
    x = (rng.standard_normal((n, k)) * sig).astype(np.float32)
    x[rng.random((n, k)) < 0.05] = 0.0
    x[rng.random((n, k)) < 0.01] = np.inf
    w = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    w[rng.random((n, k)) < 0.01] = 0x7FC3
    w[rng.random((n, k)) < 0.01] = 0x0005
    t = w12.encode(w)
    assert np.array_equal(w12.decode(t), w)
    # window rule by exhaustive search over every base
    e = ((w >> 7) & 0xFF).astype(np.int64)
    normal = (e >= 1) & (e <= 254)
    for c in range(n):
        counts = [int(np.sum(normal[c] & (e[c] >= b) & (e[c] <= b + 15))) for b in range(1, 240)]
        best = 1 + int(np.argmax(counts))
        assert int(t.base[c]) == best
        assert t.esc_ptr[c + 1] - t.esc_ptr[c] == k - counts[best - 1]


def _closed_form_bpw(sigma: float, k: int) -> float:
    def p_window(b):  # P(2^(b-127) <= |x| < 2^(b-111)) for x ~ N(0, sigma)
        lo, hi = 2.0 ** (b - 127), 2.0 ** (b - 111)
        return erf(hi / (sigma * math.sqrt(2))) - erf(lo / (sigma * math.sqrt(2)))
    best = max(range(1, 240), key=p_window)
    esc = 1.0 - p_window(best)
    return 12.0 + 40.0 / k + 32.0 * esc, best


@pytest.mark.parametrize("k,expect", [(5120, 12.0103), (512, 12.081)])
def test_bits_per_weight_closed_form(k, expect):
    bpw_cf, best = _closed_form_bpw(0.02, k)
    assert abs(bpw_cf - expect) < 2e-3
    g = make_generator(11)
    n = 327680 // k  # same number of samples at every k
    w = bf16_bits_numpy(gen_linear_bf16(g, n, k, LinearRecipe(sigma=0.02, zero_frac=0.0,
                                                                  outlier_frac=0.0)))
    t = w12.encode(w)
    assert abs(t.bits_per_weight() - bpw_cf) < 3e-3
    assert int(np.bincount(t.base).argmax()) == best


def test_config_recipe_escape_rate():
    # 1% zeros + 0.05% outliers x1000 with per-channel sigma: about 1.06-1.10% escapes
    from synth.configs import LARGE_RECIPE
    g = make_generator(12)
    w = bf16_bits_numpy(gen_linear_bf16(g, 128, 5120, LARGE_RECIPE))
    t = w12.encode(w)
    frac = t.n_esc / w.size
    assert 0.0104 < frac < 0.0112
    assert 12.33 < t.bits_per_weight() < 12.37
