"""gpt2_clip_adamw_step_static (no allocation, static scratch) against
gpt2_clip_adamw_step on identical inputs: two calls in a row, the second on a
smaller model, each bit-identical to the context's own step."""

import numpy as np
import pytest

from gpt2_inputs import init_params
from tests.gpu_helpers import gpu_step, say, shape, warm_state

pytestmark = pytest.mark.gpu


def _state(s, seed):
    p = init_params(s, seed)
    rng = np.random.default_rng(seed + 1)
    g = {n: (1e-3 * rng.standard_normal(a.shape)).astype(np.float32) for n, a in p.items()}
    m, v = warm_state(g, seed=seed + 2)
    return p, g, m, v


def _load(st, p, g, m, v, t):
    import torch
    st.load_params(p)
    st.load_state(m, v, t)
    for n, a in st.to_dict(st.grads).items():
        a.copy_(torch.as_tensor(g[n]))


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_static_scratch_step_equals_context_step(precision):
    import torch
    cases = [(shape("gpt2-124m-L2", 2, 12, 768, 1024, 50257, 50304), 0, "clip"),
             (shape("narrow-L1", 1, 1, 64, 128, 65, 72), 5, "noclip")]
    for s, seed, mode in cases:  # the second call is on a smaller model
        say(f"static-scratch clip + AdamW {precision} {s.name} ({mode})")
        p, g, m, v = _state(s, seed)
        from oracle.gpt2 import global_norm
        n = global_norm(g)
        max_norm = 0.5 * n if mode == "clip" else 2.0 * n
        a = gpu_step(s, precision, 1, p)
        _load(a, p, g, m, v, 6)
        a.clip_adamw_step(6e-4, 0.9, 0.95, 1e-8, 0.1, max_norm)
        b = gpu_step(s, precision, 1, p)
        _load(b, p, g, m, v, 6)
        b.clip_adamw_step_static(7, 6e-4, 0.9, 0.95, 1e-8, 0.1, max_norm)
        torch.cuda.synchronize()
        assert a.sync_status() == 0 and b.sync_status() == 0
        for x, y in ((a.params, b.params), (a.m, b.m), (a.v, b.v), (a.d_norm, b.d_norm),
                     (a.d_clipped, b.d_clipped)):
            assert torch.equal(x, y)
        if precision == "bf16":
            assert torch.equal(a.params_bf16, b.params_bf16)
        assert int(b.d_clipped.item()) == (1 if mode == "clip" else 0)
        a.close()
        b.close()


def test_static_scratch_step_rejects_bad_arguments():
    from gpt_decoder_pre_amd.lib import GPT2_ERR_ARG, Gpt2Error
    s = shape("narrow-L1", 1, 1, 64, 128, 65, 72)
    st = gpu_step(s, "fp32", 1, init_params(s, 0))
    with pytest.raises(Gpt2Error) as e:
        st.clip_adamw_step_static(0, 1e-3)
    assert e.value.code == GPT2_ERR_ARG
    st.close()
