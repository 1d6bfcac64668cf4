"""GPU: the HBM stream probes (read only, write only, copy) through the C ABI,
on a size that is not a multiple of the probes' grid stride (the tail loop)
and on one shorter than a single stride."""

import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [(1 << 22) * 3 + 20, 1000])
def test_stream_probes_move_what_they_should(n):
    import torch

    from gpt_decoder_pre_amd import lib as L
    from tests.gpu_helpers import say
    say(f"stream probes, n = {n}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    x = torch.rand(n, generator=g, device=dev)
    part = torch.full((L.probe_partials(n),), float("nan"), device=dev)
    L.stream_probe(L.PROBE_READ, x, part)
    y = torch.zeros(n + 8, device=dev)
    L.stream_probe(L.PROBE_COPY, x, y)
    z = torch.zeros(n + 4, device=dev)
    L.stream_probe(L.PROBE_WRITE, None, z[:n])
    torch.cuda.synchronize()
    want = float(x.double().sum())
    got = float(part.double().sum())
    assert abs(got - want) <= 1e-5 * want
    assert torch.equal(y[:n], x) and bool((y[n:] == 0).all())
    assert bool((z[:n] == 0.5).all()) and bool((z[n:] == 0).all())
