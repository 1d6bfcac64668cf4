"""Shared helpers of the GPU tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded inputs."""

import sys

import numpy as np

from gpt2_inputs import ModelShape, init_params, micro_batches, token_stream

BF16_LOSS_ABS = 2e-2      # bf16 mode: |loss_gpu - loss_ref|
BF16_GRAD_COS = 0.99      # bf16 mode: per-tensor cosine similarity of gradients
BF16_UPDATE_REL = 2e-2    # bf16 mode: relative L2 error of the parameter update
FP32_REL = 1e-4           # fp32 mode: relative error of loss, gradients, update


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / max(na * nb, 1e-300))


def shape(name, L, NH, C, T, V, Vp):
    return ModelShape(name, L, NH, C, T, V, Vp)


def batches_for(s: ModelShape, B, T, k, kind="zipf", seed=1):
    stream = token_stream(kind, k * B * T + 1, s.vocab_size, seed)
    return micro_batches(stream, k, B, T)


def to_dev(batches):
    import torch
    x = torch.tensor(np.stack([b[0] for b in batches]), dtype=torch.int32, device="cuda")
    y = torch.tensor(np.stack([b[1] for b in batches]), dtype=torch.int32, device="cuda")
    return x, y


def gpu_step(s, precision, B, params):
    from gpt_decoder_pre_amd.lib import GPT2Step
    st = GPT2Step(s, precision, max_batch=B)
    st.load_params(params)
    return st


def host(d):
    return {n: v.detach().float().cpu().numpy().astype(np.float64) for n, v in d.items()}


def warm_state(grads_ref, seed=7):
    """A non-degenerate AdamW state (first moment ~ N(0, (g_rms/2)^2), second
    moment ~ g_rms^2 (1 + U)) so that the step is not sign-like; the same fp32
    arrays go to both paths."""
    rng = np.random.default_rng(seed)
    m, v = {}, {}
    for n, g in grads_ref.items():
        r = float(np.sqrt(np.mean(np.square(g)))) + 1e-12
        m[n] = (0.5 * r * rng.standard_normal(g.shape)).astype(np.float32)
        v[n] = ((r * r) * (1.0 + rng.random(g.shape))).astype(np.float32)
    return m, v
