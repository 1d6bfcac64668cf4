"""Pins of the loss-scaling oracle (oracle/amp.py), on the CPU: its scale
sequence and skip decisions against PyTorch's own dynamic scaler on the CPU
(the scaler the pages' fp16 AMP runs), closed forms of the growth schedule,
and planted mistakes that the pins must catch."""

import numpy as np
import pytest

from oracle import amp
from oracle import gpt2 as ref

# found_inf pattern of a run: good steps, isolated and repeated overflows
PATTERN = [0, 0, 1, 0, 0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0, 1, 0]


def _torch_run(pattern, init_scale, growth_interval):
    """PyTorch's GradScaler (CPU) over a one-tensor model, an inf planted in
    the gradient where the pattern says; returns the scale and growth counter
    after each step and whether the parameter moved."""
    import torch
    w = torch.nn.Parameter(torch.ones(4, dtype=torch.float32))
    opt = torch.optim.SGD([w], lr=0.5)
    sc = torch.amp.GradScaler("cpu", init_scale=init_scale, growth_factor=2.0, backoff_factor=0.5,
                              growth_interval=growth_interval)
    out = []
    for bad in pattern:
        opt.zero_grad()
        loss = (w * torch.arange(1.0, 5.0)).sum()
        sc.scale(loss).backward()
        if bad:
            with torch.no_grad():
                w.grad[1] = float("inf")
        before = w.detach().clone()
        sc.step(opt)
        sc.update()
        moved = not torch.equal(before, w.detach())
        out.append((float(sc.get_scale()), int(sc._growth_tracker.item()), moved))
    return out


def _oracle_run(pattern, init_scale, growth_interval, update=None):
    update = update or amp.scaler_update
    s, good, out = init_scale, 0, []
    for bad in pattern:
        s, good = update(s, good, bool(bad), growth_interval=growth_interval)
        out.append((s, good, not bad))
    return out


@pytest.mark.parametrize("interval", [1, 3, 2000])
def test_scale_sequence_matches_pytorch_grad_scaler(interval):
    pytest.importorskip("torch")
    want = _torch_run(PATTERN, 1024.0, interval)
    got = _oracle_run(PATTERN, 1024.0, interval)
    assert got == want


def test_growth_closed_form():
    """n good steps from S0: S0 * 2^(n // interval), counter n % interval."""
    for n in range(0, 25):
        for interval in (1, 4, 7):
            s, good = 8.0, 0
            for _ in range(n):
                s, good = amp.scaler_update(s, good, False, growth_interval=interval)
            assert s == 8.0 * 2.0 ** (n // interval) and good == n % interval


def test_defaults_are_pytorchs():
    torch = pytest.importorskip("torch")
    sc = torch.amp.GradScaler("cpu")
    assert (amp.INIT_SCALE, amp.GROWTH_FACTOR, amp.BACKOFF_FACTOR, amp.GROWTH_INTERVAL) == \
        (sc.get_scale(), sc.get_growth_factor(), sc.get_backoff_factor(), sc.get_growth_interval())


def _toy_step_fn(params, m, v, t, grads):
    return ref.adamw(params, grads, m, v, t, lr=1e-3)


def _toy_state():
    rng = np.random.default_rng(3)
    p = {"w": rng.standard_normal((3, 4)), "b": rng.standard_normal(4)}
    g = {n: rng.standard_normal(a.shape) for n, a in p.items()}
    z = {n: np.zeros_like(a) for n, a in p.items()}
    return p, g, z


def test_good_step_is_the_unscaled_step():
    p, g, z = _toy_state()
    S = 2.0 ** 12
    scaled = {n: a * S for n, a in g.items()}
    p2, m2, v2, t2, s2, good2, skipped = amp.amp_step(p, z, z, 4, scaled, S, 5, _toy_step_fn)
    want_p, want_m, want_v = ref.adamw(p, g, z, z, 5, lr=1e-3)
    assert not skipped and t2 == 5 and s2 == S and good2 == 6
    for n in p:
        np.testing.assert_array_equal(p2[n], want_p[n])
        np.testing.assert_array_equal(m2[n], want_m[n])


def test_overflow_skips_and_backs_off():
    p, g, z = _toy_state()
    scaled = {n: a.copy() for n, a in g.items()}
    scaled["b"][2] = np.inf
    p2, m2, v2, t2, s2, good2, skipped = amp.amp_step(p, z, z, 4, scaled, 1024.0, 5, _toy_step_fn)
    assert skipped and t2 == 4 and s2 == 512.0 and good2 == 0
    assert p2 is p and m2 is z and v2 is z
    scaled["b"][2] = np.nan
    assert amp.amp_step(p, z, z, 4, scaled, 1024.0, 5, _toy_step_fn)[6]


def _no_reset(scale, good, found_inf, growth_factor=2.0, backoff_factor=0.5, growth_interval=2000):
    """Planted: an overflow backs off but keeps counting good steps."""
    if found_inf:
        return scale * backoff_factor, good
    good += 1
    if good >= growth_interval:
        return scale * growth_factor, 0
    return scale, good


def _grow_one_late(scale, good, found_inf, growth_factor=2.0, backoff_factor=0.5, growth_interval=2000):
    """Planted: growth after interval + 1 good steps."""
    if found_inf:
        return scale * backoff_factor, 0
    good += 1
    if good > growth_interval:
        return scale * growth_factor, 0
    return scale, good


@pytest.mark.parametrize("bad", [_no_reset, _grow_one_late])
def test_planted_scaler_mistake_is_caught(bad):
    pytest.importorskip("torch")
    want = _torch_run(PATTERN, 1024.0, 3)
    assert _oracle_run(PATTERN, 1024.0, 3, update=bad) != want
