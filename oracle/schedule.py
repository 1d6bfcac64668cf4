"""fp64 oracle of the learning-rate schedule of the training loop.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Linear warmup to the peak rate, then a half-cosine decay to the floor, then
the floor (AxonLM README, "Key Features": cosine LR + warmup; "Training
Recipe": peak 6e-4, minimum 6e-5 = peak / 10, 715 warmup steps, 19,073 total
steps; GPT From Scratch, "Architecture diagram": warmup + cosine LR).  The
pages name the schedule but print no formula; the reading taken: step s
counts optimizer steps from 0, the warmup rate is peak (s + 1) / warmup (so
the last warmup step runs at the peak), and the decay's phase runs from 0 at
s = warmup to pi at s = total.
"""

from __future__ import annotations

import math


def lr_at(step, max_lr, min_lr, warmup_steps, max_steps):
    if step < warmup_steps:
        return max_lr * (step + 1) / warmup_steps
    if step > max_steps:
        return min_lr
    phase = math.pi * (step - warmup_steps) / (max_steps - warmup_steps)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + math.cos(phase))
