"""Cross-check of the oracle against PyTorch library routines on the CPU, fp64.

PyTorch's own LayerNorm, tanh-GELU, causal scaled-dot-product attention,
cross-entropy, autograd, clip_grad_norm_ and AdamW (the routines the pages'
recipes call) are an independent implementation of the same definitions.
They share no code with the oracle or the HIP path.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from gpt2_inputs import ModelShape, init_params, micro_batches, uniform_tokens
from oracle import gpt2 as ref


def torch_loss(P, x, y, n_head):
    B, T = x.shape
    C = P["wte"].shape[1]
    L = P["qkv_w"].shape[0]
    h = P["wte"][x] + P["wpe"][:T]
    for l in range(L):
        a = F.layer_norm(h, (C,), P["ln1_w"][l], P["ln1_b"][l], eps=1e-5)
        qkv = F.linear(a, P["qkv_w"][l], P["qkv_b"][l] if "qkv_b" in P else None)
        q, k, v = qkv.split(C, dim=-1)
        q, k, v = (t.view(B, T, n_head, C // n_head).transpose(1, 2) for t in (q, k, v))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.transpose(1, 2).reshape(B, T, C)
        h = h + F.linear(o, P["proj_w"][l], P["proj_b"][l])
        a = F.layer_norm(h, (C,), P["ln2_w"][l], P["ln2_b"][l], eps=1e-5)
        u = F.gelu(F.linear(a, P["fc_w"][l], P["fc_b"][l]), approximate="tanh")
        h = h + F.linear(u, P["fcproj_w"][l], P["fcproj_b"][l])
    h = F.layer_norm(h, (C,), P["lnf_w"], P["lnf_b"], eps=1e-5)
    z = h @ (P["lm_head"] if "lm_head" in P else P["wte"]).T
    return F.cross_entropy(z.reshape(B * T, -1), y.reshape(-1))


def _setup(seed=0, L=2, NH=4, C=32, T=16, V=29, B=3, tied=True, qkv_bias=True):
    s = ModelShape("xcheck", L, NH, C, T, V, V, tied=tied, qkv_bias=qkv_bias)
    p = init_params(s, seed)
    rng = np.random.default_rng(seed + 100)
    for n in p:  # exercise biases and LN parameters
        if n.endswith("_b") or n.startswith("ln"):
            p[n] = (p[n] + 0.05 * rng.standard_normal(p[n].shape)).astype(np.float32)
    (x, y), = micro_batches(uniform_tokens(B * T + 1, V, seed + 1), 1, B, T)
    return s, p, x, y


def test_forward_and_gradients_match_torch_autograd():
    _autograd_case(True, True)


def test_untied_variant_matches_torch_autograd():
    """The variant with its own lm_head and no QKV bias (Genesis "Model Specs")."""
    _autograd_case(False, False)


def _autograd_case(tied, qkv_bias):
    s, p, x, y = _setup(tied=tied, qkv_bias=qkv_bias)
    assert ("lm_head" in p) == (not tied) and ("qkv_b" in p) == qkv_bias
    P = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in p.items()}
    lt = torch_loss(P, torch.tensor(x, dtype=torch.long), torch.tensor(y, dtype=torch.long),
                    s.n_head)
    lt.backward()
    lo, go = ref.loss_and_grads(p, x, y, s.n_head)
    assert abs(lo - lt.item()) < 1e-12
    for n in p:
        want = P[n].grad.numpy()
        err = np.linalg.norm(go[n] - want) / max(np.linalg.norm(want), 1e-300)
        assert err < 1e-10, (n, err)


@pytest.mark.parametrize("max_norm_mode", ["clip", "noclip"])
def test_clip_and_adamw_match_torch(max_norm_mode):
    s, p, x, y = _setup(seed=3)
    lo, go = ref.loss_and_grads(p, x, y, s.n_head)
    n = ref.global_norm(go)
    max_norm = 0.5 * n if max_norm_mode == "clip" else 2.0 * n
    lr, wd = 1e-3, 0.1

    # torch: parameters per tensor (one per block and name), groups by rank
    tensors, names = [], []
    for name, a in p.items():
        if name in ref.BLOCK_NAMES:
            for l in range(a.shape[0]):
                tensors.append(torch.tensor(a[l], dtype=torch.float64))
                names.append((name, l))
        else:
            tensors.append(torch.tensor(a, dtype=torch.float64))
            names.append((name, None))
    for t, (name, l) in zip(tensors, names):
        g = go[name] if l is None else go[name][l]
        t.grad = torch.tensor(g, dtype=torch.float64)
    tn = torch.nn.utils.clip_grad_norm_(tensors, max_norm)
    groups = [{"params": [t for t in tensors if t.dim() >= 2], "weight_decay": wd},
              {"params": [t for t in tensors if t.dim() < 2], "weight_decay": 0.0}]
    opt = torch.optim.AdamW(groups, lr=lr, betas=(0.9, 0.95), eps=1e-8, foreach=False)
    # two optimizer steps on the same gradients exercise the moments and t = 2
    opt.step()
    for t in tensors:
        t.grad = t.grad.clone()
    opt.step()

    norm, clipped, cg = ref.clip_by_global_norm(go, max_norm)
    assert abs(norm - tn.item()) < 1e-12 * norm
    assert clipped == (max_norm_mode == "clip")
    zero = {k: np.zeros(a.shape) for k, a in p.items()}
    P1, M1, V1 = ref.adamw(p, cg, zero, zero, 1, lr, 0.9, 0.95, 1e-8, wd)
    P2, _, _ = ref.adamw(P1, cg, M1, V1, 2, lr, 0.9, 0.95, 1e-8, wd)
    for t, (name, l) in zip(tensors, names):
        want = t.detach().numpy()
        got = P2[name] if l is None else P2[name][l]
        assert np.max(np.abs(got - want)) < 1e-13, name


def _torch_tensors(p):
    """One fp64 torch tensor per block and name (the per-tensor view the
    optimizer groups act on), with the (name, layer) key of each."""
    tensors, names = [], []
    for name, a in p.items():
        if name in ref.BLOCK_NAMES:
            for l in range(a.shape[0]):
                tensors.append(torch.tensor(a[l], dtype=torch.float64))
                names.append((name, l))
        else:
            tensors.append(torch.tensor(a, dtype=torch.float64))
            names.append((name, None))
    return tensors, names


def _pick(d, name, l):
    return d[name] if l is None else d[name][l]


@pytest.mark.parametrize("max_norm_mode", ["clip", "noclip"])
def test_train_step_matches_torch_accumulate_clip_adamw(max_norm_mode):
    """The whole oracle step (accumulate over two micro-batches, clip, AdamW
    from a warm state at t = 4) against torch autograd + clip_grad_norm_ +
    AdamW with per-tensor parameter groups.  With max_norm = 0.5 n the clip
    fires, so AdamW fed the unclipped gradients or a wrong t would differ."""
    s, p, x, y = _setup(seed=5, B=4)
    batches = [(x[:2], y[:2]), (x[2:], y[2:])]
    _, g_probe = ref.accumulate(p, batches, s.n_head)
    n = ref.global_norm(g_probe)
    max_norm = 0.5 * n if max_norm_mode == "clip" else 2.0 * n
    lr, wd, t_prev = 1e-3, 0.1, 3
    rng = np.random.default_rng(11)
    m0 = {k: 0.1 * rng.standard_normal(a.shape) * np.sqrt(np.mean(g_probe[k] ** 2)) for k, a in p.items()}
    v0 = {k: (1.0 + rng.random(a.shape)) * np.mean(g_probe[k] ** 2) for k, a in p.items()}

    r = ref.train_step(p, m0, v0, t_prev + 1, batches, s.n_head, lr=lr, weight_decay=wd, max_norm=max_norm)
    # the same step from a precomputed accumulation takes the same path after it
    r2 = ref.train_step(p, m0, v0, t_prev + 1, None, s.n_head, lr=lr, weight_decay=wd, max_norm=max_norm,
                        accumulated=ref.accumulate(p, batches, s.n_head))
    for k in ("params", "m", "v"):
        for name in p:
            assert np.array_equal(r[k][name], r2[k][name]), (k, name)

    # torch: loss of each micro-batch / k through autograd, summed gradients
    P = {k: torch.tensor(a, dtype=torch.float64, requires_grad=True) for k, a in p.items()}
    total = 0.0
    for bx, by in batches:
        lt = torch_loss(P, torch.tensor(bx, dtype=torch.long), torch.tensor(by, dtype=torch.long),
                        s.n_head) / len(batches)
        lt.backward()
        total += lt.item()
    grads = {k: P[k].grad.numpy() for k in p}
    tensors, names = _torch_tensors(p)
    for tt, (name, l) in zip(tensors, names):
        tt.grad = torch.tensor(_pick(grads, name, l), dtype=torch.float64)
    tn = torch.nn.utils.clip_grad_norm_(tensors, max_norm)
    groups = [{"params": [tt for tt in tensors if tt.dim() >= 2], "weight_decay": wd},
              {"params": [tt for tt in tensors if tt.dim() < 2], "weight_decay": 0.0}]
    opt = torch.optim.AdamW(groups, lr=lr, betas=(0.9, 0.95), eps=1e-8, foreach=False)
    for tt, (name, l) in zip(tensors, names):
        opt.state[tt] = {"step": torch.tensor(float(t_prev)),
                         "exp_avg": torch.tensor(_pick(m0, name, l), dtype=torch.float64),
                         "exp_avg_sq": torch.tensor(_pick(v0, name, l), dtype=torch.float64)}
    opt.step()

    assert abs(r["loss"] - total) < 1e-12
    assert abs(r["norm"] - tn.item()) < 1e-12 * r["norm"]
    assert r["clipped"] == (max_norm_mode == "clip")
    for tt, (name, l) in zip(tensors, names):
        st = opt.state[tt]
        assert np.max(np.abs(_pick(r["params"], name, l) - tt.detach().numpy())) < 1e-13, (name, l)
        assert np.max(np.abs(_pick(r["m"], name, l) - st["exp_avg"].numpy())) < 1e-13, (name, l)
        assert np.max(np.abs(_pick(r["v"], name, l) - st["exp_avg_sq"].numpy())) < 1e-15, (name, l)
        # the returned gradients are the accumulated (pre-clip) ones
        assert np.max(np.abs(_pick(r["grads"], name, l) - _pick(grads, name, l))) < 1e-13, (name, l)
