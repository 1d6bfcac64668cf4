"""The training loop around the GPT-2 step: warmup + cosine learning rate,
sequential batches from token shard files, periodic checkpoints and
auto-resume from the latest one, and a CSV log (step, loss, lr, norm,
tokens/s).

    python -m gpt_decoder_pre_amd.train --config gpt2-124m --data shard0.bin shard1.bin \\
        --steps 19073 --ckpt-dir checkpoints --ckpt-every 500

Every step of the path runs behind the C ABI: the loader (gpt2_loader_*),
the schedule (gpt2_lr_at), gpt2_accumulate, gpt2_clip_adamw_step and the
checkpoints (gpt2_checkpoint_*).  This module only sequences the calls.
"""

from __future__ import annotations

import argparse
import glob
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CKPT_RE = re.compile(r"step_(\d{8})\.ckpt$")


def latest_checkpoint(ckpt_dir):
    """The checkpoint of the highest step in ckpt_dir, or None."""
    best = None
    for p in glob.glob(os.path.join(ckpt_dir, "step_*.ckpt")):
        m = CKPT_RE.search(p)
        if m and (best is None or int(m.group(1)) > best[0]):
            best = (int(m.group(1)), p)
    return best[1] if best else None


class Trainer:
    """One GPT2Step context, one loader and the schedule."""

    def __init__(self, run, paths, dtype="uint16", max_lr=6e-4, min_lr=6e-5, warmup=715, max_steps=19073,
                 ckpt_dir=None, ckpt_every=0, log_path=None, device="cuda:0"):
        import torch

        from gpt2_inputs import init_params
        from gpt_decoder_pre_amd.lib import GPT2Step, TokenLoader, lr_at
        self.torch = torch
        self.run = run
        s = run.shape
        k, B, T = run.grad_accum, run.micro_batch, run.seq_len
        self.step = GPT2Step(s, run.precision, max_batch=B, device=device)
        self.step.load_params(init_params(s, run.seed_weights))
        self.loader = TokenLoader(paths, s.vocab_size, k, B, T, dtype=dtype)
        self.sched = (max_lr, min_lr, warmup, max_steps)
        self.lr_at = lr_at
        self.x = torch.empty((k, B, T), dtype=torch.int32, device=self.step.device)
        self.y = torch.empty_like(self.x)
        self.ckpt_dir = ckpt_dir
        self.ckpt_every = ckpt_every
        self.log = open(log_path, "a") if log_path else None
        if self.log and self.log.tell() == 0:
            self.log.write("step,loss,lr,norm,clipped,tokens_per_s\n")

    @property
    def t(self):
        """Optimizer steps taken (the AdamW step counter)."""
        return self.step.step_count()

    def save(self, path):
        self.step.checkpoint_save(path, self.loader.state())

    def resume(self, path):
        sh, pos = self.step.checkpoint_load(path)[:2]
        self.loader.seek(sh, pos)

    def train_step(self):
        """One optimizer step; returns (loss, lr, norm, clipped)."""
        r = self.run
        lr = self.lr_at(*self.sched, self.t)
        self.loader.next_device(self.x, self.y, self.step.stream)
        loss = self.step.accumulate(self.x, self.y)
        norm, clipped = self.step.clip_adamw_step(lr, r.beta1, r.beta2, r.eps, r.weight_decay, r.max_norm)
        return loss, lr, norm, clipped

    def train(self, n_steps, log_every=1):
        torch = self.torch
        r = self.run
        tokens = r.grad_accum * r.micro_batch * r.seq_len
        for _ in range(n_steps):
            t0 = time.perf_counter()
            loss, lr, norm, clipped = self.train_step()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            if self.step.sync_status() != 0:
                raise RuntimeError(f"device error at step {self.t}")
            t = self.t
            if self.log and t % log_every == 0:
                self.log.write(f"{t},{loss.item():.6f},{lr:.6e},{norm.item():.6f},{int(clipped.item())},"
                               f"{tokens / dt:.1f}\n")
                self.log.flush()
            if self.ckpt_dir and self.ckpt_every and t % self.ckpt_every == 0:
                os.makedirs(self.ckpt_dir, exist_ok=True)
                self.save(os.path.join(self.ckpt_dir, f"step_{t:08d}.ckpt"))

    def close(self):
        if self.log:
            self.log.close()
        self.loader.close()
        self.step.close()


def main(argv=None):
    from gpt2_inputs import RUNS
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="gpt2-124m", choices=sorted(RUNS))
    ap.add_argument("--data", nargs="+", required=True, help="token shard files")
    ap.add_argument("--dtype", default="uint16", choices=["uint16", "int32"])
    ap.add_argument("--steps", type=int, default=100, help="optimizer steps to run in this invocation")
    ap.add_argument("--max-lr", type=float, default=6e-4)
    ap.add_argument("--min-lr", type=float, default=6e-5)
    ap.add_argument("--warmup", type=int, default=715)
    ap.add_argument("--max-steps", type=int, default=19073)
    ap.add_argument("--ckpt-dir", default=None)
    ap.add_argument("--ckpt-every", type=int, default=500)
    ap.add_argument("--no-resume", action="store_true", help="ignore checkpoints in --ckpt-dir")
    ap.add_argument("--log", default=None, help="CSV log file (appended)")
    a = ap.parse_args(argv)
    tr = Trainer(RUNS[a.config], a.data, a.dtype, a.max_lr, a.min_lr, a.warmup, a.max_steps, a.ckpt_dir,
                 a.ckpt_every, a.log)
    if a.ckpt_dir and not a.no_resume:
        p = latest_checkpoint(a.ckpt_dir)
        if p:
            tr.resume(p)
            print(f"resumed from {p} at step {tr.t}", flush=True)
    tr.train(a.steps)
    print(f"done: step {tr.t}", flush=True)
    tr.close()


if __name__ == "__main__":
    main()
