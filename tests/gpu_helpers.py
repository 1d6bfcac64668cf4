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


# ---------------------------------------------------------------- per tensor ----

def per_tensor(d):
    """(name, layer) -> array: one entry per tensor as the model defines them
    (the stacked per-block arrays split by layer; layer None for the global
    tensors), so that a gate over one layer is not diluted by the others."""
    from oracle.gpt2 import BLOCK_NAMES
    out = {}
    for n, a in d.items():
        if n in BLOCK_NAMES:
            for l in range(a.shape[0]):
                out[(n, l)] = a[l]
        else:
            out[(n, None)] = a
    return out


# ---------------------------------------------------- oracle on many threads ----

def _seq_loss_grads_dx0(params, x, y, n_head, scale):
    from oracle import gpt2 as ref
    loss, cache = ref.forward(params, x, y, n_head, loss_scale=scale)
    g = ref.backward(params, cache)
    return loss, g, cache["dx0"]


_SEQ_MEMO = {}


def _digest(params, x, y, n_head):
    import hashlib
    h = hashlib.blake2b(digest_size=16)
    for n in sorted(params):
        h.update(n.encode())
        h.update(np.ascontiguousarray(params[n]).tobytes())
    h.update(np.ascontiguousarray(x).tobytes())
    h.update(np.ascontiguousarray(y).tobytes())
    h.update(str(n_head).encode())
    return h.hexdigest()


def oracle_accumulate_per_sequence(params, x, y, n_head, workers=None, with_dx0=False, memo=False):
    """The oracle's accumulation with every sequence of the (B, T) batch as its
    own micro-batch (loss scale 1/B): equal to the one batch of B sequences
    (the accumulation pin).  The sequences run on a thread pool (numpy
    releases the GIL inside its loops and BLAS calls) with single-threaded
    BLAS: concurrent calls into a multi-threaded OpenBLAS from several
    threads return corrupted products.  The sums are taken in sequence order.
    Returns (mean loss, grads).  With memo, the result is kept for the rest
    of the session under a digest of (params, x, y, n_head), so two tests of
    the same batch share one oracle run (the caller must not modify it)."""
    if memo:
        key = (_digest(params, x, y, n_head), with_dx0)
        if key not in _SEQ_MEMO:
            _SEQ_MEMO[key] = oracle_accumulate_per_sequence(params, x, y, n_head, workers, with_dx0)
        return _SEQ_MEMO[key]
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B = x.shape[0]
    cpus = min(16, len(os.sched_getaffinity(0)))
    workers = workers or max(1, min(B, cpus))
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda b: _seq_loss_grads_dx0(params, x[b:b + 1], y[b:b + 1], n_head, 1.0 / B),
                                  range(B)))
    total = 0.0
    grads = None
    for loss, g, _ in results:  # fixed order: sequence 0, 1, ...
        total += loss
        if grads is None:
            grads = g
        else:
            for n in grads:
                grads[n] += g[n]
    if with_dx0:
        return total, grads, np.concatenate([r[2] for r in results], axis=0)
    return total, grads


def oracle_warm_state(params, s, B, T, steps=10, seed=101, lr=6e-4, kind="zipf"):
    """A warm AdamW state from the oracle itself: `steps` fp64 oracle training
    steps from m = v = 0 on other seeded batches.  Returns (params, m, v, t)
    cast to fp32, to be loaded identically into both paths."""
    from oracle import gpt2 as ref
    p = {n: np.asarray(a, np.float64) for n, a in params.items()}
    m = {n: np.zeros(a.shape) for n, a in p.items()}
    v = {n: np.zeros(a.shape) for n, a in p.items()}
    stream = token_stream(kind, steps * B * T + 1, s.vocab_size, seed)
    for t in range(1, steps + 1):
        (bx, by), = micro_batches(stream[(t - 1) * B * T:t * B * T + 1], 1, B, T)
        r = ref.train_step(p, m, v, t, [(bx, by)], s.n_head, lr=lr)
        p, m, v = r["params"], r["m"], r["v"]
    f32 = lambda d: {n: np.asarray(a, np.float32) for n, a in d.items()}  # noqa: E731
    return f32(p), f32(m), f32(v), steps
