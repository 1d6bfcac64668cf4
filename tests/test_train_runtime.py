"""The training-loop runtime on the CPU: the learning-rate schedule against
its oracle and the recipe's numbers, and the token loader's windows against
plain slicing of the token stream (index work: bit-exact)."""

import math
import os

import numpy as np
import pytest

from gpt_decoder_pre_amd import lib as L
from oracle import schedule as sched

RECIPE = dict(max_lr=6e-4, min_lr=6e-5, warmup_steps=715, max_steps=19073)  # AxonLM "Training Recipe"


def test_oracle_schedule_recipe_values():
    r = RECIPE
    f = lambda s: sched.lr_at(s, **r)  # noqa: E731
    assert f(0) == pytest.approx(6e-4 / 715, rel=1e-15)
    assert f(714) == pytest.approx(6e-4, rel=1e-15)          # the peak at the last warmup step
    assert f(715) == pytest.approx(6e-4, rel=1e-15)          # the decay starts at the peak
    mid = 715 + (19073 - 715) // 2
    assert f(mid) == pytest.approx(0.5 * (6e-4 + 6e-5), rel=1e-9)  # half way down the cosine
    assert f(19073) == pytest.approx(6e-5, rel=1e-15)
    assert f(10 ** 6) == 6e-5
    # linear warmup, then strictly decreasing
    w = [f(s) for s in range(715)]
    assert np.allclose(np.diff(w), 6e-4 / 715, rtol=1e-9)
    d = [f(s) for s in range(715, 19074, 97)]
    assert all(a > b for a, b in zip(d, d[1:]))


def test_library_schedule_matches_oracle():
    for s in list(range(0, 800, 7)) + list(range(715, 19200, 311)) + [19073, 19074, 10 ** 7]:
        want = sched.lr_at(s, **RECIPE)
        got = L.lr_at(RECIPE["max_lr"], RECIPE["min_lr"], RECIPE["warmup_steps"], RECIPE["max_steps"], s)
        assert abs(got - want) <= 1e-15 * want, (s, got, want)


def test_library_schedule_rejects_bad_arguments():
    assert math.isnan(L.lr_at(6e-4, 6e-5, 0, 10, 1))
    assert math.isnan(L.lr_at(6e-4, 6e-5, 10, 10, 1))
    assert math.isnan(L.lr_at(6e-4, 6e-5, 10, 100, -1))


def _write(path, ids, dtype):
    np.asarray(ids, dtype=np.uint16 if dtype == "uint16" else np.int32).tofile(path)


@pytest.mark.parametrize("dtype", ["uint16", "int32"])
def test_loader_windows_are_sequential_and_cross_shards(tmp_path, dtype):
    rng = np.random.default_rng(0)
    k, B, T, V = 2, 3, 8, 500
    n = k * B * T
    shards = [rng.integers(0, V, size=s) for s in (3 * n + 5, n - 3, 2 * n + 1)]  # the middle one is too short
    paths = []
    for i, a in enumerate(shards):
        p = str(tmp_path / f"s{i}.bin")
        _write(p, a, dtype)
        paths.append(p)
    ld = L.TokenLoader(paths, V, k, B, T, dtype=dtype)
    # expected: windows of n + 1 ids at 0, n, 2n of shard 0, then shard 2 at 0, n, then shard 0 again
    expect = [(0, 0), (0, n), (0, 2 * n), (2, 0), (2, n), (0, 0)]
    for sh, pos in expect:
        assert ld.state() == (sh, pos)
        x, y = ld.next_host()
        w = shards[sh][pos:pos + n + 1]
        assert np.array_equal(x.reshape(-1), w[:-1])
        assert np.array_equal(y.reshape(-1), w[1:])
        # micro-batch i is the i-th block of B x T ids of the window
        assert np.array_equal(x[1], w[B * T:2 * B * T].reshape(B, T))
    ld.seek(2, n)
    x, _ = ld.next_host()
    assert np.array_equal(x.reshape(-1), shards[2][n:2 * n])
    with pytest.raises(L.Gpt2Error) as e:
        ld.seek(1, 0)  # no whole window fits there
    assert e.value.code == L.GPT2_ERR_ARG
    ld.close()


def test_loader_errors(tmp_path):
    k, B, T, V = 1, 2, 4, 100
    small = str(tmp_path / "small.bin")
    _write(small, np.arange(k * B * T), "uint16")  # one id short of a window
    with pytest.raises(L.Gpt2Error) as e:
        L.TokenLoader([small], V, k, B, T)
    assert e.value.code == L.GPT2_ERR_BATCH  # the data is too small for one batch
    with pytest.raises(L.Gpt2Error) as e:
        L.TokenLoader([str(tmp_path / "missing.bin")], V, k, B, T)
    assert e.value.code == L.GPT2_ERR_IO
    odd = str(tmp_path / "odd.bin")
    open(odd, "wb").write(b"\x00" * 7)  # not a whole number of int32 ids
    with pytest.raises(L.Gpt2Error) as e:
        L.TokenLoader([odd], V, k, B, T, dtype="int32")
    assert e.value.code == L.GPT2_ERR_IO
    bad = str(tmp_path / "bad.bin")
    ids = np.arange(3 * k * B * T) % V
    ids[k * B * T + 2] = V  # an id outside the vocabulary in the second window
    _write(bad, ids, "uint16")
    ld = L.TokenLoader([bad], V, k, B, T)
    ld.next_host()
    with pytest.raises(L.Gpt2Error) as e:
        ld.next_host()
    assert e.value.code == L.GPT2_ERR_TOKEN
    assert ld.state() == (0, k * B * T)  # the loader did not advance past the bad window
    ld.close()
