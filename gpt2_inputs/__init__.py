"""Seeded synthetic inputs for one GPT-2 pre-training step.

This module is the only code shared by the fp64 oracle (``oracle/``) and the
GPU path's tests and benchmark. It holds model shapes, the initial parameter
draw and token streams, and nothing of the step's arithmetic (no layer norm,
attention, loss, gradient or optimizer code).

Sources (the pages are GPT-2 pre-training write-ups):
  * model scales 12/12/768, 24/16/1024, 36/20/1280, 48/25/1600 -- AxonLM
    README, "Model Scales" table;
  * char-level toy defaults (4 layers, 4 heads, 128 dims, block 64) and the
    vocabulary padded from 50,257 to 50,304 -- "GPT From Scratch", "Problem"
    and "Key decisions";
  * init N(0, 0.02) with residual projections scaled by 1/sqrt(2L) --
    AxonLM README, "Key Features" (weight init scaling);
  * batches are consecutive windows of one token stream, target = next
    token -- "GPT From Scratch", architecture diagram (sequential batches).
"""

from .configs import (  # noqa: F401
    ModelShape,
    RunConfig,
    SHAPES,
    RUNS,
    param_shapes,
    per_layer_names,
    n_params,
)
from .generators import (  # noqa: F401
    init_params,
    uniform_tokens,
    zipf_tokens,
    zipf_probabilities,
    token_stream,
    micro_batches,
)
