"""The training loop on the GPU: loader-fed steps, checkpoint / resume (the
resumed step equals the uninterrupted one bit for bit), and the loss falling
under the warmup + cosine schedule."""

import os

import numpy as np
import pytest

from gpt2_inputs import RUNS, RunConfig, token_stream
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _shards(tmp_path, n_ids, vocab, seed, kind="uniform", parts=2):
    ids = token_stream(kind, n_ids, vocab, seed)
    paths = []
    for i, a in enumerate(np.array_split(ids, parts)):
        p = str(tmp_path / f"shard{i}.bin")
        a.astype(np.uint16).tofile(p)
        paths.append(p)
    return paths


def _toy_run(k=2):
    r = RUNS["toy"]
    return RunConfig("toy-k", r.shape, 4, k, 64, "fp32", "uniform", 1e-3)


@pytest.mark.parametrize("precision", ["fp32", "bf16", "fp16"])
def test_checkpoint_resume_is_bitwise(tmp_path, precision):
    import torch

    from gpt_decoder_pre_amd.train import Trainer, latest_checkpoint
    if precision == "fp32":
        run = _toy_run()
    else:
        from tests.gpu_helpers import shape
        s = shape("gpt2-124m-L1", 1, 12, 768, 1024, 50257, 50304)
        run = RunConfig("l1", s, 2, 2, 128, precision, "zipf", 6e-4)
    say(f"checkpoint / resume {precision}")
    s = run.shape
    paths = _shards(tmp_path, 9 * run.tokens_per_step, s.vocab_size, 3, kind=run.tokens)
    sched = dict(max_lr=1e-3, min_lr=1e-4, warmup=2, max_steps=6)
    ck = str(tmp_path / "ck")
    a = Trainer(run, paths, ckpt_dir=ck, ckpt_every=3, **sched)
    a.train(5)
    torch.cuda.synchronize()
    want = [t.clone() for t in (a.step.params, a.step.m, a.step.v)]
    want_scaler = a.step.loss_scaler_state()[:2] if precision == "fp16" else None
    a.close()
    p = latest_checkpoint(ck)
    assert p.endswith("step_00000003.ckpt") and not os.path.exists(p + ".tmp")
    b = Trainer(run, paths, **sched)
    b.resume(p)
    assert b.t == 3
    b.train(2)
    torch.cuda.synchronize()
    assert b.t == 5
    for x, y in zip(want, (b.step.params, b.step.m, b.step.v)):
        assert torch.equal(x, y)
    if precision == "fp16":  # the loss scaler came back with the checkpoint
        assert b.step.loss_scaler_state()[:2] == want_scaler
    # a checkpoint of another model is refused
    from gpt_decoder_pre_amd.lib import GPT2_ERR_ARG, GPT2Step, Gpt2Error
    from gpt2_inputs import ModelShape
    other = GPT2Step(ModelShape("toy-2l", 2, 4, 128, 64, 65, 65), "fp32", 1)
    with pytest.raises(Gpt2Error) as e:
        other.checkpoint_load(p)
    assert e.value.code == GPT2_ERR_ARG
    other.close()
    b.close()


def test_loader_device_copy_equals_host_windows(tmp_path):
    import torch

    from gpt_decoder_pre_amd.lib import TokenLoader
    say("loader device copy")
    k, B, T, V = 3, 4, 64, 50257
    paths = _shards(tmp_path, 10 * k * B * T, V, 5, kind="zipf", parts=3)
    a = TokenLoader(paths, V, k, B, T)
    b = TokenLoader(paths, V, k, B, T)
    x = torch.empty((k, B, T), dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    st = torch.cuda.current_stream()
    for _ in range(7):  # crosses shards and reuses both staging buffers
        a.next_device(x, y, st)
        hx, hy = b.next_host()
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy(), hx) and np.array_equal(y.cpu().numpy(), hy)
    a.close()
    b.close()


def test_loss_falls_under_the_schedule(tmp_path):
    """Twenty steps of the toy model on a repeating 2-window stream: the
    loss falls well below ln 65 (the stream is memorisable)."""
    import math

    from gpt_decoder_pre_amd.train import Trainer
    run = _toy_run(k=1)
    say("loss falls under warmup + cosine")
    paths = _shards(tmp_path, 2 * run.tokens_per_step + 1, 65, 11, parts=1)
    log = str(tmp_path / "log.csv")
    tr = Trainer(run, paths, max_lr=3e-3, min_lr=3e-4, warmup=3, max_steps=20, log_path=log)
    tr.train(20)
    tr.close()
    rows = [l.split(",") for l in open(log).read().splitlines()[1:]]
    loss = [float(r[1]) for r in rows]
    lr = [float(r[2]) for r in rows]
    say(f"  loss {loss[0]:.4f} -> {loss[-1]:.4f}")
    assert len(rows) == 20
    assert abs(loss[0] - math.log(65)) < 0.1
    assert loss[-1] < loss[0] - 0.5
    assert lr[2] == pytest.approx(3e-3) and lr[-1] == pytest.approx(3e-4 + 2.7e-3 * 0.5 * (1 + math.cos(math.pi * 16 / 17)))
