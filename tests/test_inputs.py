"""The seeded input generators: init statistics, Zipf law, stream windows."""

import math

import numpy as np

from gpt2_inputs import SHAPES, init_params, micro_batches, zipf_probabilities, zipf_tokens
from gpt2_inputs import param_shapes


def test_zipf_normaliser_and_head_probability():
    p = zipf_probabilities(50257, 1.1)
    H = np.sum(np.arange(1, 50258, dtype=np.float64) ** -1.1)
    assert abs(H - 7.1969) < 1e-3
    assert abs(p[0] - 1.0 / H) < 1e-15
    assert abs(p[1] / p[0] - 2 ** -1.1) < 1e-12


def test_zipf_draws_follow_the_law():
    n = 200_000
    ids = zipf_tokens(n, 50257, seed=1)
    assert ids.min() >= 0 and ids.max() < 50257
    p = zipf_probabilities(50257, 1.1)
    for r in (0, 1, 9):
        f = np.mean(ids == r)
        sd = math.sqrt(p[r] * (1 - p[r]) / n)
        assert abs(f - p[r]) < 5 * sd
    # same seed, same stream
    assert np.array_equal(ids[:100], zipf_tokens(100, 50257, seed=1))


def test_windows_are_consecutive_and_shifted():
    s = np.arange(3 * 2 * 5 + 1, dtype=np.int32)
    mb = micro_batches(s, 3, 2, 5)
    assert len(mb) == 3
    for i, (x, y) in enumerate(mb):
        assert np.array_equal(y, x + 1)
        assert x[0, 0] == i * 10


def test_init_statistics():
    s = SHAPES["toy"]
    p = init_params(s, 0)
    assert list(p) == list(param_shapes(s))
    assert abs(p["fc_w"].std() - 0.02) < 0.001
    assert abs(p["proj_w"].std() - 0.02 / math.sqrt(2 * s.n_layer)) < 0.0005
    assert abs(p["fcproj_w"].std() - 0.02 / math.sqrt(2 * s.n_layer)) < 0.0005
    assert np.all(p["ln1_w"] == 1) and np.all(p["qkv_b"] == 0)
    q = init_params(s, 0)
    assert all(np.array_equal(p[n], q[n]) for n in p)
