"""Pins of the decoding and sampling oracle (CPU): greedy is the first
arg-max; the inverse CDF gives every kept token exactly its probability
mass; top-k and top-p keep what PyTorch's sort-based filtering keeps;
temperature sharpens the distribution as p^(1/T); decoding step i sees the
logits of the whole sequence so far."""

import numpy as np
import pytest
import torch

from gpt2_inputs import ModelShape, init_params, uniform_tokens
from oracle import generate as gen
from oracle import gpt2 as ref


def _mass(row, V, temperature, top_k, top_p, grid=20000):
    """Fraction of a fine uniform grid of u that picks each token."""
    u = (np.arange(grid) + 0.5) / grid
    picks = np.array([gen.sample(row, V, temperature, top_k, top_p, x) for x in u])
    return np.bincount(picks, minlength=V) / grid


def test_greedy_is_first_argmax():
    row = np.array([0.1, 2.0, -1.0, 2.0, 0.5])
    assert gen.sample(row, 5, 0.0, 0, 1.0, 0.3) == 1
    assert gen.sample(row, 5, 1.0, 1, 1.0, 0.99) == 1
    assert gen.sample(np.r_[row, 9.0], 5, 0.0, 0, 1.0, 0.0) == 1  # padded columns are never tokens


def test_inverse_cdf_gives_each_token_its_probability():
    rng = np.random.default_rng(0)
    row = rng.standard_normal(7) * 1.5
    p = np.exp(row - row.max())
    p /= p.sum()
    assert np.allclose(_mass(row, 7, 1.0, 0, 1.0), p, atol=2e-4)
    # in column order: u below p[0] picks column 0
    assert gen.sample(row, 7, 1.0, 0, 1.0, 0.999 * p[0]) == 0
    assert gen.sample(row, 7, 1.0, 0, 1.0, 1.001 * p[0]) == 1


def test_temperature_sharpens_as_power():
    rng = np.random.default_rng(1)
    row = rng.standard_normal(6)
    for T in (0.5, 2.0):
        q = np.exp(row / T - (row / T).max())
        q /= q.sum()
        assert np.allclose(_mass(row, 6, T, 0, 1.0), q, atol=2e-4)


def _torch_filter(row, k, p):
    """PyTorch sort-based top-k / top-p filtering (the usual formulation):
    logits below the k-th largest set to -inf; then sorted probabilities whose
    cumulative mass before them already reaches p removed."""
    z = torch.tensor(row, dtype=torch.float64)
    if k > 0:
        v, _ = torch.topk(z, k)
        z = torch.where(z < v[-1], torch.tensor(float("-inf"), dtype=z.dtype), z)
    if 0 < p < 1:
        sz, si = torch.sort(z, descending=True)
        cp = torch.cumsum(torch.softmax(sz, 0), 0)
        drop = (cp - torch.softmax(sz, 0)) >= p  # mass before this token already reaches p
        z[si[drop]] = float("-inf")
    return torch.isfinite(z).numpy()


@pytest.mark.parametrize("k,p", [(5, 1.0), (40, 1.0), (0, 0.9), (0, 0.5), (20, 0.8)])
def test_top_k_top_p_keep_what_sort_based_filtering_keeps(k, p):
    rng = np.random.default_rng(7)
    for _ in range(20):
        row = rng.standard_normal(300) * 2.0
        kept = gen.filtered_probs(row, 300, 1.0, k, p) > 0
        assert np.array_equal(kept, _torch_filter(row, k, p))


def test_top_k_keeps_ties_at_the_kth_value():
    row = np.array([3.0, 1.0, 2.0, 2.0, 0.0])
    kept = gen.filtered_probs(row, 5, 1.0, 2, 1.0) > 0
    assert kept.tolist() == [True, False, True, True, False]


def test_decoding_sees_the_whole_sequence_so_far():
    s = ModelShape("dec", 2, 2, 16, 16, 23, 24)
    p = init_params(s, 3)
    prompt = uniform_tokens(2 * 5, 23, 4).reshape(2, 5)
    u = np.random.default_rng(5).random((6, 2))
    toks, logits = gen.generate(p, prompt, 6, s.n_head, 23, 1.0, 0, 1.0, u)
    seq = np.concatenate([prompt, toks], axis=1)
    z = ref.logits(p, seq, s.n_head)
    for i in range(6):
        assert np.allclose(logits[:, i], z[:, 4 + i], rtol=0, atol=1e-12)
        for b in range(2):
            assert toks[b, i] == gen.sample(z[b, 4 + i], 23, 1.0, 0, 1.0, u[i, b])
