"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the pins catch each of them."""

import math

import numpy as np
import pytest

from oracle import gpt2 as ref
from tests import test_oracle_pins as pins
from tests import test_oracle_torch as xcheck


def _ln_unbiased(x, w, b, eps=ref.LN_EPS):
    mean = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, ddof=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, (xhat, rstd)


def _ln_bwd_dropped_term(dy, w, cache):
    xhat, rstd = cache
    C = dy.shape[-1]
    dxhat = dy * w
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).reshape(-1, C).sum(0), dy.reshape(-1, C).sum(0)


def _attn_one_future_key(q, k, v):
    """Off-by-one mask: query i also sees key i + 1."""
    hd, T = q.shape[-1], q.shape[-2]
    S = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    S = np.where(np.triu(np.ones((T, T), bool), k=2), -np.inf, S)
    S = S - S.max(-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(-1, keepdims=True)
    return P @ v, P


def _attn_wrong_scale(q, k, v):
    hd, T = q.shape[-1], q.shape[-2]
    S = (q @ np.swapaxes(k, -1, -2)) / hd
    S = np.where(np.triu(np.ones((T, T), bool), k=1), -np.inf, S)
    S = S - S.max(-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(-1, keepdims=True)
    return P @ v, P


def _gelu_bad_const(u):
    return 0.5 * u * (1.0 + np.tanh(ref.GELU_K * (u + 0.0447 * u ** 3)))


def _decay_everything(name, arr):
    return True


def _run_all_pins():
    """Run the cheap pins; return True if every one passes."""
    checks = [
        xcheck.test_forward_and_gradients_match_torch_autograd,
        xcheck.test_untied_variant_matches_torch_autograd,
        lambda: xcheck.test_clip_and_adamw_match_torch("clip"),
        lambda: xcheck.test_train_step_matches_torch_accumulate_clip_adamw("clip"),
        pins.test_attention_masked_equals_online_softmax_form,
        pins.test_causality_future_tokens_do_not_change_past_logits,
        pins.test_initial_loss_toy_near_ln65,
        pins.test_accumulation_equals_one_big_batch,
        pins.test_clip_closed_form,
        pins.test_adamw_first_step_closed_form,
        pins.test_layernorm_textbook_moments,
        pins.test_gelu_special_values_and_derivative,
        pins.test_zero_embedding_gives_exact_uniform_loss,
    ]
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, FloatingPointError, ValueError):
            return False
    return True


def test_unmutated_oracle_passes_all_pins():
    assert _run_all_pins()


@pytest.mark.parametrize("attr,bad", [
    ("layer_norm", _ln_unbiased),
    ("layer_norm_backward", _ln_bwd_dropped_term),
    ("causal_attention", _attn_one_future_key),
    ("causal_attention", _attn_wrong_scale),
    ("gelu", _gelu_bad_const),
    ("decays", _decay_everything),
    ("CLIP_EPS", 0.0),
    ("LN_EPS", 1e-6),
])
def test_planted_mistake_is_caught(monkeypatch, attr, bad):
    monkeypatch.setattr(ref, attr, bad)
    assert not _run_all_pins()


def test_planted_transposed_operand_in_attention_backward_is_caught(monkeypatch):
    orig = ref.causal_attention_backward

    def bad(dy, q, k, v, P):
        dq, dk, dv = orig(dy, q, k, v, P)
        scale = 1.0 / math.sqrt(q.shape[-1])
        dP = dy @ np.swapaxes(v, -1, -2)
        dS = P * (dP - (dP * P).sum(-1, keepdims=True))
        return dq, (dS @ q) * scale, dv

    monkeypatch.setattr(ref, "causal_attention_backward", bad)
    assert not _run_all_pins()


def test_planted_sign_error_in_gelu_derivative_is_caught(monkeypatch):
    orig = ref.gelu_grad
    monkeypatch.setattr(ref, "gelu_grad", lambda u: orig(u) - 2 * 0.5 * u * 0 - 0.01 * u)
    assert not _run_all_pins()


def _train_step_unclipped(params, m, v, t, batches, n_head, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                          weight_decay=0.1, max_norm=1.0, accumulated=None):
    """Plausible slip: AdamW fed the accumulated gradients instead of the clipped ones."""
    loss, grads = ref.accumulate(params, batches, n_head) if accumulated is None else accumulated
    norm, clipped, cg = ref.clip_by_global_norm(grads, max_norm)
    P, M, Vv = ref.adamw(params, grads, m, v, t, lr, beta1, beta2, eps, weight_decay)
    return {"loss": loss, "norm": norm, "clipped": clipped, "grads": grads, "params": P, "m": M, "v": Vv}


def _train_step_stale_t(params, m, v, t, batches, n_head, lr, beta1=0.9, beta2=0.95, eps=1e-8,
                        weight_decay=0.1, max_norm=1.0, accumulated=None):
    """Plausible slip: bias correction with the previous step number."""
    loss, grads = ref.accumulate(params, batches, n_head) if accumulated is None else accumulated
    norm, clipped, cg = ref.clip_by_global_norm(grads, max_norm)
    P, M, Vv = ref.adamw(params, cg, m, v, t - 1, lr, beta1, beta2, eps, weight_decay)
    return {"loss": loss, "norm": norm, "clipped": clipped, "grads": grads, "params": P, "m": M, "v": Vv}


@pytest.mark.parametrize("bad", [_train_step_unclipped, _train_step_stale_t])
def test_planted_mistake_in_train_step_wiring_is_caught(monkeypatch, bad):
    monkeypatch.setattr(ref, "train_step", bad)
    assert not _run_all_pins()


def test_planted_tied_head_in_untied_backward_is_caught(monkeypatch):
    """Plausible slip: the untied variant's backward still sends the head's
    gradient to wte."""
    monkeypatch.setattr(ref, "head_name", lambda params: "wte")
    assert not _run_all_pins()
