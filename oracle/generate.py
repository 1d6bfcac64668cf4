"""fp64 oracle of autoregressive decoding and of the sampler.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Decoding (GPT From Scratch, "Architecture diagram": GPT.generate with
temperature and top-k; Genesis model card, "Key Implementation Details":
temperature, top-k and top-p sampling): the logits of the next token are the
last position's logits of the full forward pass over the sequence so far
(``gpt2.forward``), recomputed from scratch at every step -- the plain
definition that a key / value cache must reproduce.

Sampling of one token from a row of logits over the real vocabulary
[0, vocab_size) (padded columns are never tokens):
  * temperature <= 0 or top_k == 1: the first largest logit;
  * z = logits / temperature;
  * top_k > 0: keep the columns with z at least the k-th largest z (ties at
    the k-th value kept);
  * p = softmax over the kept columns;
  * 0 < top_p < 1: sort the kept p in decreasing order, take the shortest
    prefix whose mass reaches top_p, and keep every column with p at least
    the smallest p of that prefix (ties kept);
  * the token is the first column, in column order, at which the running
    sum of the kept p exceeds u times their total, u in [0, 1) given.
The pages name the filters but not their tie rules or the order of the
inverse CDF; these are the readings taken.
"""

from __future__ import annotations

import numpy as np

from . import gpt2


def next_logits(params, idx, n_head):
    """(B, Vp) logits of the position after the last of idx (B, T)."""
    return gpt2.logits(params, np.asarray(idx), n_head)[:, -1, :]


def filtered_probs(logits_row, vocab_size, temperature, top_k, top_p):
    """The kept probabilities (unnormalised weights, zero where dropped) of
    one row; the normalisation is left to the caller."""
    z = np.asarray(logits_row, np.float64)[:vocab_size] / temperature
    keep = np.ones(vocab_size, bool)
    if 0 < top_k < vocab_size:
        kth = np.sort(z)[::-1][top_k - 1]
        keep &= z >= kth
    e = np.where(keep, np.exp(z - z[keep].max()), 0.0)
    if 0.0 < top_p < 1.0:
        order = np.argsort(-e, kind="stable")
        csum = np.cumsum(e[order])
        n = int(np.searchsorted(csum, top_p * e.sum(), side="left")) + 1
        thr = e[order[min(n, vocab_size) - 1]]
        e = np.where(e >= thr, e, 0.0)
    return e


def sample(logits_row, vocab_size, temperature, top_k, top_p, u):
    """The token chosen for one row with uniform u."""
    row = np.asarray(logits_row, np.float64)[:vocab_size]
    if temperature <= 0 or top_k == 1:
        return int(np.argmax(row))  # argmax returns the first largest
    e = filtered_probs(row, vocab_size, temperature, top_k, top_p)
    c = np.cumsum(e)
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    if i >= vocab_size or e[i] == 0.0:  # at the total itself: the last kept column
        i = int(np.nonzero(e)[0][-1])
    return i


def generate(params, prompt, n_new, n_head, vocab_size, temperature, top_k, top_p, uniforms):
    """Tokens and per-step logits of n_new decoding steps from prompt (B, T):
    step i samples from the logits of the sequence so far with uniforms[i]
    (B values), then appends the token."""
    seq = np.asarray(prompt)
    logits, tokens = [], []
    for i in range(n_new):
        z = next_logits(params, seq, n_head)
        t = np.array([sample(z[b], vocab_size, temperature, top_k, top_p, uniforms[i][b])
                      for b in range(seq.shape[0])], np.int64)
        logits.append(z)
        tokens.append(t)
        seq = np.concatenate([seq, t[:, None]], axis=1)
    return np.stack(tokens, 1), np.stack(logits, 1)
