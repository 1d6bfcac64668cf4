"""Pins of the fp64 oracle against what the pages and mathematics fix.

Every test here runs on the CPU.  Each pin is chosen so that a plausible slip
in the oracle (a dropped term, a wrong sign or index, a transposed operand)
breaks at least one of them; ``test_oracle_mutations.py`` plants such slips
and checks that they are caught.
"""

import json
import math
import os

import numpy as np
import pytest

from gpt2_inputs import ModelShape, SHAPES, init_params, micro_batches, n_params, param_shapes
from gpt2_inputs import uniform_tokens
from oracle import gpt2 as ref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def tiny(L=2, NH=2, C=16, T=8, V=11, name="tiny"):
    return ModelShape(name, L, NH, C, T, V, V)


def toy_batch(shape, B, T, seed=1, k=1):
    s = uniform_tokens(k * B * T + 1, shape.vocab_size, seed)
    return micro_batches(s, k, B, T)


# ---------------------------------------------------------------- shapes ----

def test_param_count_124m_matches_page():
    s = SHAPES["gpt2-124m"]
    s50257 = ModelShape("x", s.n_layer, s.n_head, s.n_embd, s.block_size, 50257, 50257)
    assert n_params(s50257) == GOLDEN["params_124m_vocab_50257"]["value"]


def test_param_count_untied_163m_cross_check():
    # Genesis: same 12/12/768/1024 model with its own (untied) lm_head and no
    # bias on the QKV projection.
    s = ModelShape("x", 12, 12, 768, 1024, 50257, 50257)
    untied = n_params(s) + 50257 * 768 - 12 * 3 * 768
    assert untied == GOLDEN["params_untied_163m"]["value"]


def test_param_count_of_the_untied_variant_matches_page():
    # the variant's own tensor table (lm_head added, qkv_b removed) at vocab 50,257
    s = ModelShape("x", 12, 12, 768, 1024, 50257, 50257, tied=False, qkv_bias=False)
    assert n_params(s) == GOLDEN["params_untied_163m"]["value"]
    names = list(param_shapes(s))
    assert "qkv_b" not in names and names[-1] == "lm_head"


@pytest.mark.parametrize("scale", ["small", "medium", "large", "xl"])
def test_scale_param_counts_near_page_figures(scale):
    L, NH, C = GOLDEN["scales"]["value"][scale]
    approx = GOLDEN["scales"]["approx_params"][scale]
    s = ModelShape(scale, L, NH, C, 1024, 50257, 50257)
    assert abs(n_params(s) - approx) / approx < 0.005


def test_checkpoint_size_consistent_with_fp32_params_and_two_moments():
    # 12 bytes per parameter (fp32 p, m, v) at ~124M gives the ~1.49 GB checkpoint.
    s = ModelShape("x", 12, 12, 768, 1024, 50257, 50257)
    assert abs(12 * n_params(s) - GOLDEN["checkpoint_bytes_124m"]["value"]) < 0.01e9


def test_decay_split_at_124m():
    s = SHAPES["gpt2-124m"]
    fake = {n: np.broadcast_to(np.float32(0), shp) for n, shp in param_shapes(s).items()}
    (nd, pd), (nn, pn) = ref.tensor_groups(fake)
    assert (nd, pd) == (50, 124_354_560)
    assert (nn, pn) == (98, 121_344)
    assert pd + pn == n_params(s)


# ------------------------------------------------------------- forward ----

def test_initial_loss_toy_near_ln65():
    s = SHAPES["toy"]
    p = init_params(s, 0)
    (x, y), = toy_batch(s, 4, 64)
    loss, _ = ref.forward(p, x, y, s.n_head)
    assert abs(loss - math.log(65)) < 0.1


@pytest.mark.slow
def test_initial_loss_124m_near_ln_vocab():
    s = SHAPES["gpt2-124m"]
    p = init_params(s, 0)
    (x, y), = toy_batch(ModelShape("v", 1, 1, 1, 1, 50257, 50257), 1, 32)
    loss, _ = ref.forward(p, x, y, s.n_head)
    assert abs(loss - math.log(50304)) < 0.3


def test_zero_embedding_gives_exact_uniform_loss():
    s = tiny(V=13)
    p = init_params(s, 3)
    p["wte"][:] = 0
    (x, y), = toy_batch(s, 2, 8)
    loss, cache = ref.forward(p, x, y, s.n_head)
    assert np.all(cache["logits"] == 0)
    assert abs(loss - math.log(13)) < 1e-14


def test_causality_future_tokens_do_not_change_past_logits():
    s = tiny(L=2, NH=2, C=16, T=8, V=11)
    p = init_params(s, 5)
    (x, y), = toy_batch(s, 2, 8)
    z0 = ref.logits(p, x, s.n_head)
    for t in (0, 3, 7):
        x2 = x.copy()
        x2[:, t] = (x2[:, t] + 1) % s.vocab_size
        z1 = ref.logits(p, x2, s.n_head)
        assert np.array_equal(z0[:, :t], z1[:, :t])
        assert not np.allclose(z0[:, t], z1[:, t])


def test_attention_masked_equals_online_softmax_form():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((2, 3, 37, 8)) for _ in range(3))
    y0, P = ref.causal_attention(q, k, v)
    y1, lse = ref.causal_attention_online(q, k, v, block=5)
    tol = GOLDEN["attention_equivalence_tol"]["value"]
    assert np.max(np.abs(y0 - y1)) < tol * 1e-6
    # rows of P are distributions with nothing above the diagonal
    assert np.allclose(P.sum(-1), 1.0)
    assert np.all(np.triu(P[0, 0], 1) == 0)
    # log-sum-exp is consistent with P: P[i, j] = exp(s_ij - lse_i)
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(8)
    assert np.allclose(P[..., 5, :6], np.exp(s[..., 5, :6] - lse[..., 5:6]))


def test_attention_first_position_returns_value():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 2, 6, 4)) for _ in range(3))
    y, _ = ref.causal_attention(q, k, v)
    assert np.allclose(y[:, :, 0], v[:, :, 0])
    y1, _ = ref.causal_attention(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    assert np.allclose(y1, v[:, :, :1])


def test_attention_uniform_scores_average_values():
    # q = 0 gives equal scores: position i averages v[0..i]
    rng = np.random.default_rng(2)
    v = rng.standard_normal((1, 1, 7, 3))
    z = np.zeros_like(v)
    y, _ = ref.causal_attention(z, rng.standard_normal(v.shape), v)
    for i in range(7):
        assert np.allclose(y[0, 0, i], v[0, 0, :i + 1].mean(0))


def test_layernorm_textbook_moments():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)) * 0.01 + 3.0
    y, _ = ref.layer_norm(x, np.ones(64), np.zeros(64))
    var = x.var(-1)
    assert np.allclose(y.mean(-1), 0, atol=1e-12)
    assert np.allclose(y.var(-1), var / (var + ref.LN_EPS), rtol=1e-10)


def test_gelu_special_values_and_derivative():
    u = np.linspace(-6, 6, 241)
    g = ref.gelu(u)
    assert ref.gelu(np.array(0.0)) == 0.0
    assert np.allclose(g - ref.gelu(-u), u, atol=1e-12)      # odd part is u/2
    assert abs(ref.gelu(np.array(10.0)) - 10.0) < 1e-12
    assert abs(ref.gelu(np.array(-10.0))) < 1e-12
    # the exact GELU x*Phi(x) differs from the tanh form by < 1e-3 (Hendrycks & Gimpel)
    from scipy.special import ndtr
    assert np.max(np.abs(g - u * ndtr(u))) < 1e-3
    h = 1e-5
    fd = (ref.gelu(u + h) - ref.gelu(u - h)) / (2 * h)
    assert np.max(np.abs(fd - ref.gelu_grad(u))) < 1e-8


def test_cross_entropy_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    s = tiny()
    p = init_params(s, 7)
    (x, y), = toy_batch(s, 2, 8, seed=4)
    loss, cache = ref.forward(p, x, y, s.n_head)
    z = cache["logits"]
    want = np.mean(logsumexp(z, axis=-1) - np.take_along_axis(z, y[..., None], -1)[..., 0])
    assert abs(loss - want) < 1e-13


# ------------------------------------------------------------ backward ----

def _flat_fd(shape, p, x, y, eps=1e-4):
    """Central differences of the loss for every parameter element."""
    p64 = {n: a.astype(np.float64) for n, a in p.items()}
    out = {}
    for n, a in p64.items():
        g = np.zeros_like(a)
        flat = a.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp, _ = ref.forward(p64, x, y, shape.n_head)
            flat[i] = old - eps
            lm, _ = ref.forward(p64, x, y, shape.n_head)
            flat[i] = old
            g.reshape(-1)[i] = (lp - lm) / (2 * eps)
        out[n] = g
    return out


@pytest.mark.slow
def test_backward_matches_central_differences_2layer_16dim():
    s = tiny(L=2, NH=2, C=16, T=8, V=11)
    p = init_params(s, 11)
    # non-trivial LayerNorm gains and biases so their gradients are exercised
    rng = np.random.default_rng(12)
    for n in p:
        if n.endswith("_b") or n.startswith("ln"):
            p[n] = (p[n] + 0.1 * rng.standard_normal(p[n].shape)).astype(np.float32)
    (x, y), = toy_batch(s, 2, 8, seed=13)
    _, g = ref.loss_and_grads(p, x, y, s.n_head)
    fd = _flat_fd(s, p, x, y)
    for n in p:
        err = np.linalg.norm(g[n] - fd[n]) / max(np.linalg.norm(fd[n]), 1e-30)
        assert err < 1e-6, (n, err)


def test_accumulation_equals_one_big_batch():
    s = tiny(L=2, NH=2, C=16, T=8, V=11)
    p = init_params(s, 21)
    batches = toy_batch(s, 2, 8, seed=22, k=3)
    loss_k, g_k = ref.accumulate(p, batches, s.n_head)
    X = np.concatenate([b[0] for b in batches])
    Y = np.concatenate([b[1] for b in batches])
    loss_1, g_1 = ref.loss_and_grads(p, X, Y, s.n_head)
    tol = GOLDEN["accumulation_equivalence_tol"]["value"]
    assert abs(loss_k - loss_1) < tol
    for n in p:
        assert np.max(np.abs(g_k[n] - g_1[n])) < tol * max(1.0, np.max(np.abs(g_1[n])))


def test_loss_scale_scales_loss_and_every_gradient():
    s = tiny()
    p = init_params(s, 23)
    (x, y), = toy_batch(s, 2, 8, seed=24)
    l1, g1 = ref.loss_and_grads(p, x, y, s.n_head)
    l2, g2 = ref.loss_and_grads(p, x, y, s.n_head, loss_scale=0.25)
    assert abs(l2 - 0.25 * l1) < 1e-14
    for n in p:
        assert np.allclose(g2[n], 0.25 * g1[n], rtol=1e-12, atol=1e-18)


def test_embedding_gather_and_scatter_are_exact():
    s = tiny(V=11)
    p = init_params(s, 25)
    p["wpe"][:] = 0
    (x, y), = toy_batch(s, 2, 8, seed=26)
    _, cache = ref.forward(p, x, y, s.n_head)
    assert np.array_equal(cache["x0"], p["wte"].astype(np.float64)[x])
    # the scatter part of dwte: rows of absent ids get only the lm_head part
    g = ref.backward(p, cache)
    dz_part = np.zeros_like(g["wte"])
    # recompute the lm_head part independently: dwte_head = dz^T hf
    N = x.size
    z = cache["logits"].reshape(N, -1)
    pr = np.exp(z - z.max(-1, keepdims=True))
    pr /= pr.sum(-1, keepdims=True)
    pr[np.arange(N), y.reshape(-1)] -= 1
    dz_part = (pr / N).T @ cache["hf"].reshape(N, -1)
    scatter = g["wte"] - dz_part
    absent = np.setdiff1d(np.arange(s.vocab_size), x)
    assert np.allclose(scatter[absent], 0, atol=1e-15)
    present = np.unique(x)
    want = np.zeros_like(scatter)
    np.add.at(want, x.reshape(-1), cache["dx0"].reshape(N, -1))
    assert np.allclose(scatter[present], want[present], atol=1e-14)


# ---------------------------------------------------------- optimizer ----

def test_clip_closed_form():
    rng = np.random.default_rng(30)
    g = {"a": rng.standard_normal((4, 5)), "b": rng.standard_normal(7)}
    n = math.sqrt(np.sum(g["a"] ** 2) + np.sum(g["b"] ** 2))
    norm, clipped, cg = ref.clip_by_global_norm(g, 1.0)
    assert abs(norm - n) < 1e-12 and clipped
    assert abs(ref.global_norm(cg) - 1.0 * n / (n + 1e-6)) < 1e-12
    norm, clipped, cg = ref.clip_by_global_norm(g, 2 * n)
    assert not clipped and all(np.array_equal(cg[k], g[k]) for k in g)


def test_adamw_first_step_closed_form():
    # t = 1: m_hat = g and v_hat = g^2, so dp = -lr (wd p [2-D only] + g / (|g| + eps))
    rng = np.random.default_rng(31)
    p = {"wte": rng.standard_normal((3, 4)), "lnf_b": rng.standard_normal(4)}
    g = {n: rng.standard_normal(a.shape) for n, a in p.items()}
    z = {n: np.zeros_like(a) for n, a in p.items()}
    lr, wd, eps = 1e-3, 0.1, 1e-8
    P, M, V = ref.adamw(p, g, z, z, 1, lr, 0.9, 0.95, eps, wd)
    want_w = p["wte"] * (1 - lr * wd) - lr * g["wte"] / (np.abs(g["wte"]) + eps)
    want_b = p["lnf_b"] - lr * g["lnf_b"] / (np.abs(g["lnf_b"]) + eps)
    assert np.allclose(P["wte"], want_w, rtol=0, atol=1e-15)
    assert np.allclose(P["lnf_b"], want_b, rtol=0, atol=1e-15)
    assert np.allclose(M["wte"], 0.1 * g["wte"]) and np.allclose(V["wte"], 0.05 * g["wte"] ** 2)


def test_adamw_second_step_by_hand():
    # 1-D tensor (no decay), three elements, two steps worked by hand.
    p0 = np.array([1.0, -2.0, 0.5])
    g1 = np.array([0.1, -0.2, 0.0])
    g2 = np.array([0.3, 0.1, -0.4])
    lr, b1, b2, eps = 0.01, 0.9, 0.95, 1e-8
    z = {"lnf_w": np.zeros(3)}
    P1, M1, V1 = ref.adamw({"lnf_w": p0}, {"lnf_w": g1}, z, z, 1, lr, b1, b2, eps, 0.1)
    P2, M2, V2 = ref.adamw(P1, {"lnf_w": g2}, M1, V1, 2, lr, b1, b2, eps, 0.1)
    m1 = 0.1 * g1
    v1 = 0.05 * g1 ** 2
    p1 = p0 - lr * (m1 / 0.1) / (np.sqrt(v1 / 0.05) + eps)
    m2 = 0.9 * m1 + 0.1 * g2
    v2 = 0.95 * v1 + 0.05 * g2 ** 2
    p2 = p1 - lr * (m2 / (1 - 0.81)) / (np.sqrt(v2 / (1 - 0.9025)) + eps)
    assert np.allclose(P2["lnf_w"], p2, rtol=0, atol=1e-15)
    # element 0: explicit numbers
    assert abs(p1[0] - (1.0 - 0.01 * 0.1 / (0.1 + 1e-8))) < 1e-15


@pytest.mark.slow
def test_loss_decreases_over_steps_on_a_fixed_batch():
    s = SHAPES["toy"]
    p = init_params(s, 0)
    m = {n: np.zeros(a.shape) for n, a in p.items()}
    v = {n: np.zeros(a.shape) for n, a in p.items()}
    batches = toy_batch(s, 4, 64)
    losses = []
    for t in range(1, 21):
        r = ref.train_step(p, m, v, t, batches, s.n_head, lr=1e-3)
        losses.append(r["loss"])
        p, m, v = r["params"], r["m"], r["v"]
    assert losses[-1] < losses[0] - 0.5
    assert all(b < a for a, b in zip(losses[:5], losses[1:6]))


def test_sequence_longer_than_block_raises():
    s = tiny(T=8)
    p = init_params(s, 0)
    x = np.zeros((1, 9), np.int32)
    with pytest.raises(ValueError):
        ref.forward(p, x, x, s.n_head)
