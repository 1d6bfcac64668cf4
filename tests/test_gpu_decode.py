"""Decoding on the GPU through the C ABI (gpt2_infer.h) against the oracle:
the logits of a prefill and of every cached decoding step, the sampler's
choices on the same fp32 logits and uniforms, and the error codes."""

import numpy as np
import pytest

from gpt2_inputs import SHAPES, ModelShape, init_params, token_stream
from oracle import generate as gen
from tests.gpu_helpers import cos, gpu_step, rel, say, shape

pytestmark = pytest.mark.gpu


def _sampler_margin(row, V, temperature, top_k, top_p, u):
    """Distance of u * total from the nearest cumulative boundary of the
    oracle's kept mass, relative to the total (small: the choice is decided
    by rounding); inf for greedy."""
    if temperature <= 0 or top_k == 1:
        r = np.sort(np.asarray(row, np.float64)[:V])[::-1]
        return (r[0] - r[1]) / max(abs(r[0]), 1e-30)
    e = gen.filtered_probs(row, V, temperature, top_k, top_p)
    c = np.cumsum(e)
    return float(np.min(np.abs(c - u * c[-1])) / c[-1])


def _decode_case(s, precision, B, T, steps, temperature, top_k, top_p, tol):
    import torch

    from gpt_decoder_pre_amd.lib import Decoder
    say(f"decode {precision} {s.name}: B={B} prompt T={T} + {steps} steps (T={temperature} k={top_k} p={top_p})")
    p = init_params(s, 2)
    st = gpu_step(s, precision, 1, p)
    dec = Decoder(st, B)
    prompt = token_stream("zipf" if s.vocab_size > 1000 else "uniform", B * T, s.vocab_size, 6).reshape(B, T)
    rng = np.random.default_rng(8)
    u = rng.random((steps, B)).astype(np.float32)
    x = torch.tensor(prompt, dtype=torch.int32, device="cuda")
    z = dec.prefill(x)
    seq = prompt.copy()
    worst = (1.0, 0.0)
    for i in range(steps):
        zh = z.double().cpu().numpy()
        zr = gen.next_logits(p, seq, s.n_head)  # the oracle over the GPU's sequence so far
        for b in range(B):
            c, e = cos(zh[b], zr[b]), rel(zh[b], zr[b])
            worst = (min(worst[0], c), max(worst[1], e))
            assert e <= tol, (i, b, e)
        tok = dec.sample(z, torch.tensor(u[i], device="cuda"), temperature, top_k, top_p)
        th = tok.cpu().numpy()
        for b in range(B):
            want = gen.sample(z[b].cpu().numpy(), s.vocab_size, temperature, top_k, top_p, float(u[i, b]))
            if th[b] != want:
                assert _sampler_margin(z[b].cpu().numpy(), s.vocab_size, temperature, top_k, top_p,
                                       float(u[i, b])) < 1e-5, (i, b, th[b], want)
        seq = np.concatenate([seq, th[:, None].astype(seq.dtype)], axis=1)
        z = dec.decode(tok)
        assert dec.length() == T + i + 1
    torch.cuda.synchronize()
    assert dec.sync_status() == 0
    say(f"  worst logits cosine {worst[0]:.6f}, worst rel err {worst[1]:.2e}")
    dec.close()
    st.close()


def test_decode_fp32_toy_matches_oracle():
    _decode_case(SHAPES["toy"], "fp32", 3, 10, 12, 1.0, 0, 1.0, 1e-4)


def test_decode_fp32_toy_greedy():
    _decode_case(SHAPES["toy"], "fp32", 2, 1, 20, 0.0, 0, 1.0, 1e-4)


def test_decode_bf16_gpt2_width_sampling():
    s = shape("gpt2-124m-L2", 2, 12, 768, 1024, 50257, 50304)
    _decode_case(s, "bf16", 4, 37, 6, 0.8, 40, 0.95, 2e-2)


def test_decode_bf16_untied_variant():
    s = ModelShape("genesis-L1", 1, 12, 768, 1024, 50257, 50304, tied=False, qkv_bias=False)
    _decode_case(s, "bf16", 2, 64, 4, 1.0, 0, 0.9, 2e-2)


@pytest.mark.parametrize("L,NH,C", [(2, 12, 768), (1, 25, 1600)])
def test_decode_equals_prefill_of_the_longer_prompt(L, NH, C):
    """The cached step's logits against a prefill of the whole sequence (the
    same weights; the decoding step's own products, LayerNorms in their
    prologues and attention).  Width 1600 takes the sixteen-wave forms of the
    decoding products and several k-rounds in the MLP's output product."""
    import torch

    from gpt_decoder_pre_amd.lib import Decoder
    s = shape(f"width{C}-L{L}", L, NH, C, 1024, 50257, 50304)
    say(f"decode vs prefill of the longer prompt (bf16, C={C})")
    p = init_params(s, 4)
    st = gpu_step(s, "bf16", 1, p)
    a, b = Decoder(st, 2), Decoder(st, 2)
    seq = token_stream("zipf", 2 * 70, s.vocab_size, 9).reshape(2, 70)
    x = torch.tensor(seq, dtype=torch.int32, device="cuda")
    a.prefill(x[:, :60].contiguous())
    for j in range(60, 70):
        za = a.decode(x[:, j].contiguous())
        zb = b.prefill(x[:, :j + 1].contiguous())
        torch.cuda.synchronize()
        for r in range(2):
            assert cos(za[r].double().cpu().numpy(), zb[r].double().cpu().numpy()) > 0.9999
    a.close()
    b.close()
    st.close()


@pytest.mark.parametrize("temperature,top_k,top_p", [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9),
                                                     (1.3, 200, 0.5), (1.0, 1, 1.0)])
def test_sampler_alone_matches_oracle(temperature, top_k, top_p):
    import torch

    from gpt_decoder_pre_amd.lib import sample
    say(f"sampler alone T={temperature} k={top_k} p={top_p}")
    V, Vp, B = 50257, 50304, 32
    rng = np.random.default_rng(12)
    z = (rng.standard_normal((B, Vp)) * rng.uniform(0.5, 4.0, (B, 1))).astype(np.float32)
    z[::4, 17] += 12.0  # some rows dominated by one token
    z[1::8, 100:103] = z[1::8, 100:103].max() + 1.0  # ties at the top
    u = rng.random(B).astype(np.float32)
    out = sample(torch.tensor(z, device="cuda"), torch.tensor(u, device="cuda"), V, temperature, top_k, top_p)
    got = out.cpu().numpy()
    close = 0
    for b in range(B):
        want = gen.sample(z[b], V, temperature, top_k, top_p, float(u[b]))
        if got[b] != want:
            close += 1
            assert _sampler_margin(z[b], V, temperature, top_k, top_p, float(u[b])) < 1e-5, (b, got[b], want)
        if not (temperature <= 0 or top_k == 1):
            assert gen.filtered_probs(z[b], V, temperature, top_k, top_p)[got[b]] > 0  # a kept token
    say(f"  {B - close}/{B} equal, {close} within rounding of a boundary")



def _sampler_rows(case, rng):
    """(logits rows, vocabulary size, padded width) of one sampler path."""
    if case == "ties":  # 1500 columns share the top value: too many top-k candidates to gather
        V, Vp = 50257, 50304
        z = (rng.standard_normal((8, Vp)) * 2).astype(np.float32)
        for r in range(8):
            z[r, rng.choice(V, 1500, replace=False)] = z[r].max() + 1.0
    elif case == "few_finite":  # 30 finite logits, the rest masked to -inf
        V, Vp = 50257, 50304
        z = np.full((8, Vp), -np.inf, np.float32)
        for r in range(8):
            z[r, rng.choice(V, 30, replace=False)] = rng.standard_normal(30) * 3
    elif case == "masked":  # 30% of the vocabulary masked to -inf
        V, Vp = 50257, 50304
        z = (rng.standard_normal((8, Vp)) * 3).astype(np.float32)
        z[rng.random((8, Vp)) < 0.3] = -np.inf
    elif case == "small":  # one ragged wave of columns
        V, Vp = 100, 128
        z = (rng.standard_normal((8, Vp)) * 2).astype(np.float32)
    else:  # "ragged_wave": the second wave's range ends inside it
        V, Vp = 4097, 4104
        z = (rng.standard_normal((8, Vp)) * 2).astype(np.float32)
    return z, V, Vp


@pytest.mark.parametrize("case,temperature,top_k,top_p", [
    ("ties", 1.0, 40, 1.0), ("ties", 1.0, 40, 0.9), ("few_finite", 0.8, 40, 0.9), ("few_finite", 1.0, 0, 0.7),
    ("masked", 0.9, 50, 0.95), ("masked", 1.0, 2000, 0.5), ("small", 1.0, 80, 0.9), ("small", 1.0, 10, 1.0),
    ("small", 0.0, 0, 1.0), ("ragged_wave", 1.0, 1024, 0.8), ("ragged_wave", 1.0, 0, 1.0)])
def test_sampler_paths_match_oracle(case, temperature, top_k, top_p):
    """Each of the sampler's paths -- the gathered top-k candidates, the whole
    row when the candidates overflow or the bound is -inf, top-p over few or
    many kept columns, masked and padded columns -- against the oracle."""
    import torch

    from gpt_decoder_pre_amd.lib import sample
    say(f"sampler {case} T={temperature} k={top_k} p={top_p}")
    rng = np.random.default_rng(21)
    z, V, Vp = _sampler_rows(case, rng)
    u = rng.random(z.shape[0]).astype(np.float32)
    got = sample(torch.tensor(z, device="cuda"), torch.tensor(u, device="cuda"), V, temperature, top_k,
                 top_p).cpu().numpy()
    close = 0
    for b in range(z.shape[0]):
        want = gen.sample(z[b], V, temperature, top_k, top_p, float(u[b]))
        if got[b] != want:
            close += 1
            assert _sampler_margin(z[b], V, temperature, top_k, top_p, float(u[b])) < 1e-5, (b, got[b], want)
        if not (temperature <= 0 or top_k == 1):
            assert gen.filtered_probs(z[b], V, temperature, top_k, top_p)[got[b]] > 0  # a kept token
    say(f"  {z.shape[0] - close}/{z.shape[0]} equal, {close} within rounding of a boundary")

def test_decode_error_codes():
    import torch

    from gpt_decoder_pre_amd.lib import (GPT2_ERR_BATCH, GPT2_ERR_SEQ_TOO_LONG, GPT2_ERR_STATE, GPT2_ERR_TOKEN,
                                         Decoder, Gpt2Error)
    s = SHAPES["toy"]
    say("decode error codes")
    st = gpu_step(s, "fp32", 1, init_params(s, 0))
    dec = Decoder(st, 2)
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(Gpt2Error) as e:
        dec.B = 2
        dec.decode(tok)
    assert e.value.code == GPT2_ERR_STATE
    with pytest.raises(Gpt2Error) as e:
        dec.prefill(torch.zeros(3, 4, dtype=torch.int32, device="cuda"))
    assert e.value.code == GPT2_ERR_BATCH
    with pytest.raises(Gpt2Error) as e:
        dec.prefill(torch.zeros(1, 65, dtype=torch.int32, device="cuda"))
    assert e.value.code == GPT2_ERR_SEQ_TOO_LONG
    dec.prefill(torch.zeros(2, 63, dtype=torch.int32, device="cuda"))
    dec.decode(tok)  # position 63, the last of the block
    with pytest.raises(Gpt2Error) as e:
        dec.decode(tok)
    assert e.value.code == GPT2_ERR_SEQ_TOO_LONG
    dec.prefill(torch.full((2, 4), 65, dtype=torch.int32, device="cuda"))
    assert dec.sync_status() == GPT2_ERR_TOKEN
    assert dec.sync_status() == 0
    dec.close()
    st.close()
