"""GPU: the fp16 mode (IEEE half operands and activations, fp32 master
weights, dynamic loss scaling) through the C ABI against the fp64 oracle.

Tolerances: fp16 carries 11 significant bits against bf16's 8, over a range
that the loss scale keeps the gradients inside, so the bf16 gates (gradient
cosine >= 0.99 per tensor, update relative L2 <= 2e-2, loss within 2e-2) are
tightened by the ratio of the unit roundoffs (8x for the relative errors,
64x for 1 - cosine, a second-order quantity): loss within 5e-3, cosine >=
0.9995, update relative L2 <= 5e-3.  The loss scaler (skip on a non-finite
gradient, backoff, growth) is compared exactly with oracle.amp.
"""

import numpy as np
import pytest

from gpt2_inputs import init_params
from oracle import amp
from oracle import gpt2 as ref
from tests.gpu_helpers import (batches_for, cos, gpu_step, host, oracle_accumulate_per_sequence, per_tensor, rel, say,
                               shape, to_dev, warm_state)
from tests.test_gpu_parity import BENCH_SITE_CONFIGS, _f32, _oracle_step, _run

pytestmark = pytest.mark.gpu

FP16_LOSS_ABS = 5e-3
FP16_GRAD_COS = 0.9995
FP16_UPDATE_REL = 5e-3


def _gate_fp16(p, r, g):
    say(f"  loss gpu {g['loss']:.6f} ref {r['loss']:.6f}; norm gpu {g['norm']:.5f} ref {r['norm']:.5f}")
    assert abs(g["loss"] - r["loss"]) < FP16_LOSS_ABS
    G, RG = per_tensor(g["grads"]), per_tensor(r["grads"])
    worst = min((cos(G[k], RG[k]), k) for k in G)
    say(f"  worst gradient cosine {worst[0]:.6f} {worst[1]} over {len(G)} tensors")
    for k in G:
        assert cos(G[k], RG[k]) >= FP16_GRAD_COS, (k, cos(G[k], RG[k]))
    assert abs(g["norm"] - r["norm"]) / r["norm"] < 5e-3
    assert bool(g["clipped"]) == r["clipped"]
    P0, P1, R1 = per_tensor(p), per_tensor(g["params"]), per_tensor(_f32(r["params"]))
    worst = max((rel(P1[k] - P0[k], R1[k] - P0[k]), k) for k in P0)
    say(f"  worst update rel err {worst[0]:.5f} {worst[1]}")
    for k in P0:
        e = rel(P1[k] - P0[k], R1[k] - P0[k])
        assert e <= FP16_UPDATE_REL, (k, e)


def _fp16_case(s, B, T, k, lr=6e-4, scale=None):
    say(f"fp16 step {s.name}: L={s.n_layer} C={s.n_embd} NH={s.n_head} B={B} T={T} k={k}")
    p = init_params(s, 0)
    batches = batches_for(s, B, T, k, kind="zipf")
    loss_r, g_r = ref.accumulate(p, batches, s.n_head)
    m0, v0 = warm_state(g_r)
    r = _oracle_step(p, batches, s.n_head, m0, v0, 11, lr=lr, accumulated=(loss_r, g_r))
    g = _run(s, "fp16", p, batches, warm=(m0, v0, 10), lr=lr)
    # the GPU's gradient buffer holds the scaled gradients: unscale for the gate
    S = amp.INIT_SCALE
    g["grads"] = {n: a / S for n, a in g["grads"].items()}
    _gate_fp16(p, r, g)


def test_fp16_gpt2_small_width_two_layers():
    _fp16_case(shape("gpt2-124m-L2", 2, 12, 768, 1024, 50257, 50304), 1, 1024, 2)


def test_fp16_ragged_sequence_length():
    _fp16_case(shape("gpt2-124m-L1", 1, 12, 768, 1024, 50257, 50304), 2, 200, 1)


def test_fp16_overflow_skips_the_step_then_recovers():
    """A scale of 2^40 overflows the fp16 logit gradient (its largest entries
    are about S / (B T) = 2^33 > 65,504): the step is skipped with everything
    unchanged and the scale halved.  Then at a workable scale the step runs,
    its unscaled gradients match the oracle's, and the scaler counts it."""
    import torch
    s = shape("gpt2-124m-L1", 1, 12, 768, 1024, 50257, 50304)
    B, T = 1, 128
    p = init_params(s, 0)
    batches = batches_for(s, B, T, 1, kind="zipf")
    st = gpu_step(s, "fp16", B, p)
    x, y = to_dev(batches)
    say("fp16 overflow: scale 2^40")
    st.loss_scaler(2.0 ** 40, growth_interval=3)
    before = [t.clone() for t in (st.params, st.m, st.v, st.params_bf16)]
    st.accumulate(x, y)
    norm, _ = st.clip_adamw_step(1e-3)
    torch.cuda.synchronize()
    assert st.sync_status() == 0
    scale, good, skipped = st.loss_scaler_state()
    say(f"  after: scale 2^{np.log2(scale):.0f}, good {good}, skipped {skipped}, norm {norm.item()}")
    assert skipped == 1 and good == 0 and scale == 2.0 ** 39
    assert (scale, good) == amp.scaler_update(2.0 ** 40, 0, True, growth_interval=3)
    assert not np.isfinite(norm.item())
    assert st.step_count() == 0
    for a, b in zip(before, (st.params, st.m, st.v, st.params_bf16)):
        assert torch.equal(a, b)
    say("fp16 recovery: scale 2^10")
    st.loss_scaler(2.0 ** 10, growth_interval=3)
    loss = st.accumulate(x, y)
    torch.cuda.synchronize()
    G = {n: a / 2.0 ** 10 for n, a in host(st.to_dict(st.grads)).items()}
    st.clip_adamw_step(1e-3)
    torch.cuda.synchronize()
    scale, good, skipped = st.loss_scaler_state()
    assert skipped == 0 and good == 1 and scale == 2.0 ** 10 and st.step_count() == 1
    loss_r, g_r = ref.accumulate(p, batches, s.n_head)
    assert abs(loss.item() - loss_r) < FP16_LOSS_ABS
    Gt, Rt = per_tensor(G), per_tensor(g_r)
    worst = min((cos(Gt[k], Rt[k]), k) for k in Gt)
    say(f"  loss {loss.item():.5f} (oracle {loss_r:.5f}); worst gradient cosine {worst[0]:.6f} {worst[1]}")
    assert worst[0] >= FP16_GRAD_COS
    assert not torch.equal(before[0], st.params)
    st.close()


def test_fp16_scale_grows_after_the_interval():
    import torch
    s = shape("gpt2-124m-L1", 1, 12, 768, 1024, 50257, 50304)
    B, T = 1, 64
    p = init_params(s, 0)
    st = gpu_step(s, "fp16", B, p)
    st.loss_scaler(1024.0, growth_factor=2.0, backoff_factor=0.5, growth_interval=2)
    want = (1024.0, 0)
    for i in range(5):
        x, y = to_dev(batches_for(s, B, T, 1, kind="zipf", seed=10 + i))
        st.accumulate(x, y)
        st.clip_adamw_step(1e-4)
        torch.cuda.synchronize()
        scale, good, skipped = st.loss_scaler_state()
        want = amp.scaler_update(*want, bool(skipped), growth_interval=2)
        say(f"  step {i}: scale {scale} good {good} skipped {skipped}")
        assert skipped == 0 and (scale, good) == want
    assert st.step_count() == 5 and want == (4096.0, 1)
    st.close()


def test_fp16_training_loop_lowers_the_loss(tmp_path):
    """Twenty fp16 steps of a one-block GPT-2-width model through the training
    loop (loader, schedule, accumulation, clip + AdamW with the scaler) on a
    repeating two-window stream: the loss falls well below ln V, no step is
    skipped at the default scale, and the step count and scale follow the
    scaler's rule."""
    import math

    from gpt2_inputs import RunConfig
    from gpt_decoder_pre_amd.train import Trainer
    from tests.test_gpu_train import _shards
    s = shape("gpt2-124m-L1", 1, 12, 768, 1024, 50257, 50304)
    run = RunConfig("l1-fp16", s, 2, 1, 128, "fp16", "zipf", 6e-4)
    say("fp16 training loop")
    paths = _shards(tmp_path, 2 * run.tokens_per_step + 1, s.vocab_size, 11, kind="zipf", parts=1)
    log = str(tmp_path / "log.csv")
    tr = Trainer(run, paths, max_lr=3e-3, min_lr=3e-4, warmup=3, max_steps=20, log_path=log)
    tr.step.loss_scaler(amp.INIT_SCALE, growth_interval=8)
    tr.train(20)
    scale, good, skipped = tr.step.loss_scaler_state()
    t = tr.t
    tr.close()
    rows = [l.split(",") for l in open(log).read().splitlines()[1:]]
    loss = [float(r[1]) for r in rows]
    found = [not math.isfinite(float(r[3])) for r in rows]  # a skipped step reports a non-finite norm
    want = (amp.INIT_SCALE, 0)
    for f in found:
        want = amp.scaler_update(*want, f, growth_interval=8)
    say(f"  loss {loss[0]:.4f} -> {loss[-1]:.4f}; scale {scale}, good {good}, skipped {skipped}, t {t}, "
        f"skipped steps {sum(found)}")
    assert len(rows) == 20 and t == 20 - sum(found)
    assert (scale, good) == want and skipped == int(found[-1])
    assert sum(found) <= 2  # the default scale is workable for this model
    assert abs(loss[0] - math.log(50304)) < 0.3
    assert loss[-1] < loss[0] - 2.0


def test_fp16_xl_width():
    # C = 1600 and NH = 25: partial GEMM tiles and a 25-head attention grid in fp16
    _fp16_case(shape("gpt2-1558m-L1", 1, 25, 1600, 1024, 50257, 50304), 1, 256, 2)


def test_fp16_untied_variant_gpt2_width():
    from gpt2_inputs import ModelShape
    _fp16_case(ModelShape("genesis-L1", 1, 12, 768, 1024, 50257, 50304, tied=False, qkv_bias=False), 2, 256, 2)


def test_fp16_bench_launch_shape_two_layers():
    """The benchmarked launch shapes in fp16 (micro-batch 16 x 1024 tokens at
    GPT-2 124M width, two layers, one micro-batch, the default scale 2^16):
    every GEMM runs the benchmark's tile configuration, and the unscaled
    gradients and the update from a warm state pass the fp16 gates per layer
    and tensor against the oracle (accumulated sequence by sequence)."""
    import torch
    s = shape("gpt2-124m-L2", 2, 12, 768, 1024, 50257, 50304)
    B, T, lr = 16, 1024, 6e-4
    say(f"fp16 bench launch shape: L=2 C=768 B={B} T={T}")
    p = init_params(s, 0)
    batches = batches_for(s, B, T, 1, kind="zipf")
    g = _run(s, "fp16", p, batches, warm=None, lr=lr, sites=True)
    for site, want in BENCH_SITE_CONFIGS.items():
        got = g["sites"][site]["gemm_cfg"]
        assert got == want, (site, got, want)
    x, y = batches[0]
    loss_r, g_r, dx0 = oracle_accumulate_per_sequence(p, x, y, s.n_head, with_dx0=True, memo=True)
    gdx0 = g["dx0"].reshape(B, T, -1)  # scaled by 2^16: the cosine does not see it
    worst = min((cos(gdx0[b], dx0[b]), b) for b in range(B))
    say(f"  dx0 worst sequence cosine {worst[0]:.6f} (sequence {worst[1]})")
    assert worst[0] >= FP16_GRAD_COS
    seen = np.zeros(s.padded_vocab_size, bool)
    seen[np.unique(x)] = True
    seen[np.unique(y)] = True
    for name, rows in (("in batch", seen), ("not in batch (lm_head product only)", ~seen)):
        c = cos(g["grads"]["wte"][rows], g_r["wte"][rows])
        say(f"  wte rows {name}: cosine {c:.6f}")
        assert c >= FP16_GRAD_COS, (name, c)
    m0, v0 = warm_state(g_r)
    # the update from the warm state, on the GPU's own (scaled) gradients
    st = gpu_step(s, "fp16", B, p)
    st.load_state(m0, v0, 10)
    for n, a in st.to_dict(st.grads).items():
        a.copy_(torch.as_tensor(g["grads"][n], dtype=torch.float32))
    st.clip_adamw_step(lr, 0.9, 0.95, 1e-8, 0.1, 1.0)
    torch.cuda.synchronize()
    assert st.sync_status() == 0
    assert st.loss_scaler_state() == (amp.INIT_SCALE, 1, 0)
    g["params"] = host(st.to_dict(st.params))
    g["norm"] = float(st.d_norm.item())
    g["clipped"] = int(st.d_clipped.item())
    st.close()
    g["grads"] = {n: a / amp.INIT_SCALE for n, a in g["grads"].items()}
    r = _oracle_step(p, None, s.n_head, m0, v0, 11, lr=lr, accumulated=(loss_r, g_r))
    _gate_fp16(p, r, g)
