"""fp64 CPU oracle of one GPT-2 pre-training step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path: it reads the same fp32 parameter values and int32 token ids
(from ``gpt2_inputs``) and computes everything in numpy float64, written out
from the definitions with no blocking or fusion.

What it follows (the pages are GPT-2 pre-training write-ups):
  * model -- pre-LN decoder: wte + wpe, N x [LN -> causal self-attention ->
    residual; LN -> MLP (4x, tanh-GELU) -> residual], final LN, lm_head tied
    to wte: hanzo gpt LLM.md "GPT Model Architecture"; "GPT From Scratch"
    "Key decisions"; Genesis model card "Architecture" diagram.
  * loss -- mean softmax cross-entropy over every position, softmax over the
    whole padded vocabulary (initial loss near ln(V): "GPT From Scratch",
    "Results").
  * accumulation -- each micro-batch loss scaled by 1/k, gradients summed;
    equals one large batch ("GPT From Scratch", "Key decisions").
  * clipping -- global L2 norm over all parameters, scaled by
    max_norm / (norm + 1e-6) when that factor is below 1 (Genesis
    "Project Structure": gradient clipping; AxonLM "Training Recipe": 1.0).
  * AdamW -- decoupled decay only on tensors of two or more dimensions,
    betas (0.9, 0.95) (AxonLM "Training Recipe"; "GPT From Scratch"
    "Key decisions").

Readings where the pages are silent (the PyTorch defaults the pages' code
uses): LayerNorm eps 1e-5 with biased variance; attention scale 1/sqrt(hd)
with key j visible to query i iff j <= i; q|k|v are consecutive C-blocks of
the 3C projection and head h owns columns [h*hd, (h+1)*hd) of each; GELU is
0.5 u (1 + tanh(sqrt(2/pi)(u + 0.044715 u^3))); no dropout; AdamW eps 1e-8
with bias correction, decay p <- p (1 - lr wd) before the Adam term.
"""

from __future__ import annotations

import math
from collections import OrderedDict

import numpy as np

LN_EPS = 1e-5
GELU_K = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715
CLIP_EPS = 1e-6

GLOBAL_NAMES = ("wte", "wpe", "lnf_w", "lnf_b", "lm_head")
BLOCK_NAMES = ("ln1_w", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
               "ln2_w", "ln2_b", "fc_w", "fc_b", "fcproj_w", "fcproj_b")


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def layer_norm(x, w, b, eps=LN_EPS):
    """Per-row normalisation with biased variance, then gain and shift."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, (xhat, rstd)


def layer_norm_backward(dy, w, cache):
    """Gradients of y = xhat * w + b with xhat = (x - mean(x)) / sqrt(var(x) + eps)."""
    xhat, rstd = cache
    C = dy.shape[-1]
    dxhat = dy * w
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    dw = (dy * xhat).reshape(-1, C).sum(axis=0)
    db = dy.reshape(-1, C).sum(axis=0)
    return dx, dw, db


def gelu(u):
    """tanh form of GELU."""
    return 0.5 * u * (1.0 + np.tanh(GELU_K * (u + GELU_A * u ** 3)))


def gelu_grad(u):
    t = np.tanh(GELU_K * (u + GELU_A * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_K * (1.0 + 3.0 * GELU_A * u * u)


def causal_attention(q, k, v):
    """Masked-softmax attention, materialised in full.

    q, k, v: (B, NH, T, hd).  S = q k^T / sqrt(hd); S[i, j] = -inf for j > i;
    P = softmax over j; y = P v.  Returns (y, P).
    """
    hd = q.shape[-1]
    T = q.shape[-2]
    S = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    S = np.where(future, -np.inf, S)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=-1, keepdims=True)
    return P @ v, P


def causal_attention_online(q, k, v, block=16):
    """The same attention by blocks of keys with a running max and running sum
    (the online-softmax form of flash attention).  An independent formulation
    used only to pin ``causal_attention``.  Returns (y, lse)."""
    B, NH, T, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    y = np.zeros_like(q)
    lse = np.zeros((B, NH, T))
    for i in range(T):
        m = np.full((B, NH), -np.inf)
        l = np.zeros((B, NH))
        acc = np.zeros((B, NH, hd))
        for j0 in range(0, i + 1, block):
            j1 = min(j0 + block, i + 1)
            s = np.einsum("bhd,bhjd->bhj", q[:, :, i, :], k[:, :, j0:j1, :]) * scale
            m_new = np.maximum(m, s.max(axis=-1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[..., None])
            l = l * alpha + p.sum(axis=-1)
            acc = acc * alpha[..., None] + np.einsum("bhj,bhjd->bhd", p, v[:, :, j0:j1, :])
            m = m_new
        y[:, :, i, :] = acc / l[..., None]
        lse[:, :, i] = m + np.log(l)
    return y, lse


def causal_attention_backward(dy, q, k, v, P):
    """Backward of y = softmax(mask(q k^T / sqrt(hd))) v by the softmax Jacobian."""
    hd = q.shape[-1]
    scale = 1.0 / math.sqrt(hd)
    dv = np.swapaxes(P, -1, -2) @ dy
    dP = dy @ np.swapaxes(v, -1, -2)
    dS = P * (dP - (dP * P).sum(axis=-1, keepdims=True))
    dq = (dS @ k) * scale
    dk = (np.swapaxes(dS, -1, -2) @ q) * scale
    return dq, dk, dv


def _split_heads(x, n_head):
    B, T, C = x.shape
    return x.reshape(B, T, n_head, C // n_head).transpose(0, 2, 1, 3)


def _merge_heads(x):
    B, NH, T, hd = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, T, NH * hd)


# --------------------------------------------------------------------------
# forward + loss
# --------------------------------------------------------------------------

def head_name(params):
    """The lm_head weight: wte when tied (AxonLM "Key Features": weight
    tying), else the model's own "lm_head" (Genesis "Model Specs": the head
    kept separate from the embedding)."""
    return "lm_head" if "lm_head" in params else "wte"


def _as64(params):
    return {n: np.asarray(a, dtype=np.float64) for n, a in params.items()}


def forward(params, idx, targets, n_head, loss_scale=1.0):
    """Forward pass and mean cross-entropy.

    params: dict of arrays (per-block tensors stacked on a leading layer axis);
    idx, targets: int arrays (B, T).  Returns (loss * loss_scale, cache).
    """
    p = _as64(params)
    idx = np.asarray(idx)
    targets = np.asarray(targets)
    B, T = idx.shape
    V, C = p["wte"].shape
    if T > p["wpe"].shape[0]:
        raise ValueError(f"sequence length {T} exceeds block size {p['wpe'].shape[0]}")
    L = p["qkv_w"].shape[0]

    x = p["wte"][idx] + p["wpe"][:T][None, :, :]
    cache = {"idx": idx, "targets": targets, "x0": x, "layers": [], "n_head": n_head,
             "loss_scale": loss_scale}
    for l in range(L):
        lc = {"x_in": x}
        h1, lc["ln1"] = layer_norm(x, p["ln1_w"][l], p["ln1_b"][l])
        qkv = h1 @ p["qkv_w"][l].T
        if "qkv_b" in p:
            qkv = qkv + p["qkv_b"][l]
        q = _split_heads(qkv[..., 0:C], n_head)
        k = _split_heads(qkv[..., C:2 * C], n_head)
        v = _split_heads(qkv[..., 2 * C:3 * C], n_head)
        yh, P = causal_attention(q, k, v)
        y = _merge_heads(yh)
        x = x + y @ p["proj_w"][l].T + p["proj_b"][l]
        lc.update(h1=h1, qkv=qkv, q=q, k=k, v=v, P=P, y=y, x_mid=x)
        h2, lc["ln2"] = layer_norm(x, p["ln2_w"][l], p["ln2_b"][l])
        u = h2 @ p["fc_w"][l].T + p["fc_b"][l]
        g = gelu(u)
        x = x + g @ p["fcproj_w"][l].T + p["fcproj_b"][l]
        lc.update(h2=h2, u=u, g=g)
        cache["layers"].append(lc)
    cache["x_final"] = x
    hf, cache["lnf"] = layer_norm(x, p["lnf_w"], p["lnf_b"])
    z = hf @ p[head_name(p)].T
    cache.update(hf=hf, logits=z)

    zmax = z.max(axis=-1, keepdims=True)
    lse = (zmax + np.log(np.exp(z - zmax).sum(axis=-1, keepdims=True)))[..., 0]
    picked = np.take_along_axis(z, targets[..., None], axis=-1)[..., 0]
    per_tok = lse - picked
    cache["lse"] = lse
    cache["per_token_loss"] = per_tok
    return per_tok.mean() * loss_scale, cache


def logits(params, idx, n_head):
    z = forward(params, idx, np.zeros_like(np.asarray(idx)), n_head)[1]["logits"]
    return z


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def backward(params, cache):
    """Gradients of (mean cross-entropy * loss_scale) w.r.t. every parameter."""
    p = _as64(params)
    n_head = cache["n_head"]
    idx, targets = cache["idx"], cache["targets"]
    B, T = idx.shape
    V, C = p["wte"].shape
    L = p["qkv_w"].shape[0]
    N = B * T
    g = OrderedDict((n, np.zeros_like(a)) for n, a in p.items())

    # d(mean CE)/dz = (softmax(z) - onehot(target)) / N
    z = cache["logits"]
    dz = np.exp(z - cache["lse"][..., None])
    np.put_along_axis(dz, targets[..., None],
                      np.take_along_axis(dz, targets[..., None], axis=-1) - 1.0, axis=-1)
    dz *= cache["loss_scale"] / N

    # lm_head: z = hf W^T with W = wte (tied) or the model's own lm_head
    head = head_name(p)
    dhf = dz @ p[head]
    g[head] += dz.reshape(N, V).T @ cache["hf"].reshape(N, C)
    dx, g["lnf_w"], g["lnf_b"] = layer_norm_backward(dhf, p["lnf_w"], cache["lnf"])

    for l in reversed(range(L)):
        lc = cache["layers"][l]
        # x_out = x_mid + gelu(LN2(x_mid) Wfc^T + bfc) Wfp^T + bfp
        g["fcproj_b"][l] = dx.reshape(N, C).sum(axis=0)
        g["fcproj_w"][l] = dx.reshape(N, C).T @ lc["g"].reshape(N, 4 * C)
        dg = dx @ p["fcproj_w"][l]
        du = dg * gelu_grad(lc["u"])
        g["fc_b"][l] = du.reshape(N, 4 * C).sum(axis=0)
        g["fc_w"][l] = du.reshape(N, 4 * C).T @ lc["h2"].reshape(N, C)
        dh2 = du @ p["fc_w"][l]
        dln, g["ln2_w"][l], g["ln2_b"][l] = layer_norm_backward(dh2, p["ln2_w"][l], lc["ln2"])
        dx = dx + dln
        # x_mid = x_in + attn(LN1(x_in)) Wp^T + bp
        g["proj_b"][l] = dx.reshape(N, C).sum(axis=0)
        g["proj_w"][l] = dx.reshape(N, C).T @ lc["y"].reshape(N, C)
        dy = dx @ p["proj_w"][l]
        dq, dk, dv = causal_attention_backward(_split_heads(dy, n_head), lc["q"], lc["k"],
                                               lc["v"], lc["P"])
        dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
        if "qkv_b" in g:
            g["qkv_b"][l] = dqkv.reshape(N, 3 * C).sum(axis=0)
        g["qkv_w"][l] = dqkv.reshape(N, 3 * C).T @ lc["h1"].reshape(N, C)
        dh1 = dqkv @ p["qkv_w"][l]
        dln, g["ln1_w"][l], g["ln1_b"][l] = layer_norm_backward(dh1, p["ln1_w"][l], lc["ln1"])
        dx = dx + dln

    # x0 = wte[idx] + wpe[:T]
    np.add.at(g["wte"], idx.reshape(-1), dx.reshape(N, C))
    g["wpe"][:T] += dx.sum(axis=0)
    cache["dx0"] = dx
    return g


def loss_and_grads(params, idx, targets, n_head, loss_scale=1.0):
    loss, cache = forward(params, idx, targets, n_head, loss_scale)
    return loss, backward(params, cache)


def accumulate(params, batches, n_head):
    """k micro-batches, each loss scaled by 1/k; gradients summed.
    Returns (mean loss, grads)."""
    k = len(batches)
    total = 0.0
    grads = None
    for x, y in batches:
        loss, g = loss_and_grads(params, x, y, n_head, loss_scale=1.0 / k)
        total += loss
        if grads is None:
            grads = g
        else:
            for n in grads:
                grads[n] += g[n]
    return total, grads


# --------------------------------------------------------------------------
# clipping and AdamW
# --------------------------------------------------------------------------

def global_norm(grads):
    return math.sqrt(sum(float(np.sum(np.asarray(a, np.float64) ** 2)) for a in grads.values()))


def clip_by_global_norm(grads, max_norm):
    """Returns (norm, clipped?, clipped grads).  The factor
    max_norm / (norm + 1e-6) is applied when it is below 1."""
    norm = global_norm(grads)
    coef = max_norm / (norm + CLIP_EPS)
    clipped = coef < 1.0
    out = OrderedDict()
    for n, a in grads.items():
        a = np.asarray(a, np.float64)
        out[n] = a * coef if clipped else a.copy()
    return norm, clipped, out


def decays(name, arr):
    """Weight decay applies to tensors of two or more dimensions.  Per-block
    names are stacked on a layer axis, so their per-tensor rank is ndim - 1."""
    rank = arr.ndim - 1 if name in BLOCK_NAMES else arr.ndim
    return rank >= 2


def tensor_groups(params):
    """(decayed tensors, params), (not decayed tensors, params), one tensor
    per block and name."""
    nd = [0, 0]
    npar = [0, 0]
    for n, a in params.items():
        count = a.shape[0] if n in BLOCK_NAMES else 1
        per = a.size // count
        i = 0 if decays(n, a) else 1
        nd[i] += count
        npar[i] += per * count
    return (nd[0], npar[0]), (nd[1], npar[1])


def adamw(params, grads, m, v, t, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
    """One AdamW step (t counts from 1).  Returns new (params, m, v)."""
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    P, M, Vv = OrderedDict(), OrderedDict(), OrderedDict()
    for n in params:
        p = np.asarray(params[n], np.float64)
        gg = np.asarray(grads[n], np.float64)
        mm = beta1 * np.asarray(m[n], np.float64) + (1.0 - beta1) * gg
        vv = beta2 * np.asarray(v[n], np.float64) + (1.0 - beta2) * gg * gg
        if decays(n, p):
            p = p * (1.0 - lr * weight_decay)
        p = p - lr * (mm / bc1) / (np.sqrt(vv / bc2) + eps)
        P[n], M[n], Vv[n] = p, mm, vv
    return P, M, Vv


def train_step(params, m, v, t, batches, n_head, lr, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, max_norm=1.0, accumulated=None):
    """Accumulate over the micro-batches, clip, AdamW (t is the new step
    number).  Returns dict with loss, norm, clipped, grads, params, m, v.
    accumulated: an already computed (mean loss, grads) of the same
    micro-batches (batches is then unused)."""
    loss, grads = accumulate(params, batches, n_head) if accumulated is None else accumulated
    norm, clipped, cg = clip_by_global_norm(grads, max_norm)
    P, M, Vv = adamw(params, cg, m, v, t, lr, beta1, beta2, eps, weight_decay)
    return {"loss": loss, "norm": norm, "clipped": clipped, "grads": grads,
            "params": P, "m": M, "v": Vv}
