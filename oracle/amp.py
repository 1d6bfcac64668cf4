"""Dynamic loss scaling of the fp16 mode: the oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  Plain Python and
numpy float64; it shares no code with the HIP path.

What it follows: the Genesis model card trains with FP16 mixed precision
("Training Features": Mixed Precision (AMP) -- FP16), and the AxonLM README
notes that its bf16 AMP needs no loss scaling ("Key Features"), i.e. the fp16
one does.  The pages name PyTorch's AMP and give no constants, so the reading
is PyTorch's dynamic scaler with its defaults:

  * every backward forms the gradient of S * loss, so the accumulated
    gradients are S * g;
  * the optimizer step first unscales (g = grads / S); if any unscaled
    gradient is not finite, the step is skipped: parameters, moments and the
    step count stay as they were;
  * then the scale is updated: after a skipped step S <- S * backoff and the
    count of good steps restarts at 0; after a good one the count goes up by
    one, and when it reaches the growth interval, S <- S * growth and the
    count restarts;
  * defaults S = 2^16, growth 2, backoff 0.5, interval 2000.

The arithmetic of the step itself is that of ``oracle.gpt2.train_step`` on the
unscaled gradients (S is a power of two, so scaling and unscaling are exact in
any binary floating point without overflow or underflow).  Whether fp16
gradients overflow is a property of the fp16 arithmetic, which this fp64
oracle does not model: the skip decision enters as an input.
"""

from __future__ import annotations

import numpy as np

INIT_SCALE = 65536.0
GROWTH_FACTOR = 2.0
BACKOFF_FACTOR = 0.5
GROWTH_INTERVAL = 2000


def scaler_update(scale, good_steps, found_inf, growth_factor=GROWTH_FACTOR, backoff_factor=BACKOFF_FACTOR,
                  growth_interval=GROWTH_INTERVAL):
    """(scale, good_steps) after one optimizer step that found (or not) a
    non-finite unscaled gradient."""
    if found_inf:
        return scale * backoff_factor, 0
    good_steps += 1
    if good_steps == growth_interval:
        return scale * growth_factor, 0
    return scale, good_steps


def found_inf(scaled_grads):
    """Whether any gradient (held times the scale) is not finite."""
    return any(not np.all(np.isfinite(np.asarray(g, np.float64))) for g in scaled_grads.values())


def amp_step(params, m, v, t, scaled_grads, scale, good_steps, step_fn, **scaler_kw):
    """One optimizer step under loss scaling.  scaled_grads: the accumulated
    gradients times scale; step_fn(params, m, v, t, grads) -> (params, m, v)
    is the optimizer step (clip + AdamW) on unscaled gradients.  Returns
    (params, m, v, t, scale, good_steps, skipped)."""
    inf = found_inf(scaled_grads)
    new_scale, new_good = scaler_update(scale, good_steps, inf, **scaler_kw)
    if inf:
        return params, m, v, t, new_scale, new_good, True
    grads = {n: np.asarray(g, np.float64) / scale for n, g in scaled_grads.items()}
    p2, m2, v2 = step_fn(params, m, v, t + 1, grads)
    return p2, m2, v2, t + 1, new_scale, new_good, False
