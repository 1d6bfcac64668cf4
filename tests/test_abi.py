"""The C ABI library on the CPU: it loads, exports every function the header
declares, and its host-only queries (sizes, parameter layout, config checks)
agree with the independent shape table.  No kernel is launched here."""

import ctypes
import os
import re

import pytest

from gpt2_inputs import SHAPES, ModelShape, n_params, param_shapes
from gpt_decoder_pre_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def header_functions():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(gpt2_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from gpt_decoder_pre_amd import build
        build.build()
    return L.load_library()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert "gpt2_init" in names and "gpt2_clip_adamw_step" in names
    assert sorted(names) == sorted(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", list(SHAPES))
def test_size_query_and_layout_match_shape_table(lib, name):
    s = SHAPES[name]
    prec = "fp32" if name == "toy" else "bf16"
    cfg = L.make_config(s, prec, 2)
    sz = L.query_sizes(cfg)
    assert sz.n_params == n_params(s)
    assert sz.params_bf16_bytes == (2 * sz.n_params if prec == "bf16" else 0)
    assert sz.workspace_bytes > 0
    lay = L.tensor_layout(cfg)
    shapes = param_shapes(s)
    assert list(lay) == list(shapes)
    off = 0
    for n, (o, shp) in lay.items():
        assert o == off, n
        assert tuple(shp) == tuple(shapes[n]), n
        k = 1
        for d in shp:
            k *= d
        off += k
    assert off == sz.n_params


def test_workspace_grows_with_batch(lib):
    s = SHAPES["gpt2-124m"]
    a = L.query_sizes(L.make_config(s, "bf16", 1)).workspace_bytes
    b = L.query_sizes(L.make_config(s, "bf16", 16)).workspace_bytes
    assert b > 10 * a // 2
    assert b < 64 * 2 ** 30  # fits easily in 288 GB of HBM


@pytest.mark.parametrize("bad", [
    dict(n_embd=100),                        # C % NH != 0 with NH = 12 ... and C % 8 != 0
    dict(n_head=7),                          # 768 % 7 != 0
    dict(padded_vocab_size=50000),           # padded < vocab
    dict(max_batch=0),
    dict(precision=7),
])
def test_invalid_config_is_rejected(lib, bad):
    s = SHAPES["gpt2-124m"]
    cfg = L.make_config(s, "bf16", 2)
    for k, v in bad.items():
        setattr(cfg, k, v)
    sz = L.gpt2_sizes()
    assert lib.gpt2_init(ctypes.byref(cfg), None, None, ctypes.byref(sz), None) == L.GPT2_ERR_ARG


def test_bf16_mode_needs_head_dim_64(lib):
    cfg = L.make_config(ModelShape("x", 2, 4, 128, 64, 65, 72), "bf16", 1)  # head dim 32
    sz = L.gpt2_sizes()
    assert lib.gpt2_init(ctypes.byref(cfg), None, None, ctypes.byref(sz), None) == L.GPT2_ERR_ARG
    cfg.precision = L.GPT2_FP32
    assert lib.gpt2_init(ctypes.byref(cfg), None, None, ctypes.byref(sz), None) == L.GPT2_OK


def test_null_arguments_are_rejected_without_touching_the_gpu(lib):
    assert lib.gpt2_forward_loss(None, None, None, 1, 1, 1.0, None) == L.GPT2_ERR_ARG
    assert lib.gpt2_backward(None) == L.GPT2_ERR_ARG
    assert lib.gpt2_accumulate(None, None, None, 1, 1, 1, None) == L.GPT2_ERR_ARG
    assert lib.gpt2_clip_adamw_step(None, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, None, None) == L.GPT2_ERR_ARG
    assert lib.gpt2_get_step(None) == -1
    lib.gpt2_destroy(None)


def test_fp16_mode_sizes_and_refusals(lib):
    """The fp16 mode has the bf16 mode's layout and constraints; the entry
    point without a context and the decoding context refuse it (its loss
    scaler lives in a training context); the scaler calls refuse a NULL or
    non-fp16 context.  None of these touches the GPU."""
    s = SHAPES["gpt2-124m"]
    a = L.query_sizes(L.make_config(s, "bf16", 2))
    h = L.query_sizes(L.make_config(s, "fp16", 2))
    assert (h.n_params, h.workspace_bytes, h.params_bf16_bytes) == (a.n_params, a.workspace_bytes,
                                                                    a.params_bf16_bytes)
    cfg = L.make_config(ModelShape("x", 2, 4, 128, 64, 65, 72), "fp16", 1)  # head dim 32
    sz = L.gpt2_sizes()
    assert lib.gpt2_init(ctypes.byref(cfg), None, None, ctypes.byref(sz), None) == L.GPT2_ERR_ARG
    cfg = L.make_config(s, "fp16", 1)
    one = ctypes.c_void_p(256)  # never dereferenced: the config is refused first
    bufs = L.gpt2_buffers(one, one, one, one, one, one)
    assert lib.gpt2_clip_adamw_step_static(ctypes.byref(cfg), ctypes.byref(bufs), None, 1, 1e-3, 0.9, 0.95, 1e-8,
                                           0.1, 1.0, one, one) == L.GPT2_ERR_ARG
    isz = L.gpt2_infer_sizes()
    assert lib.gpt2_infer_init(ctypes.byref(cfg), None, None, None, None, None, ctypes.byref(isz),
                               None) == L.GPT2_ERR_ARG
    f, i = ctypes.c_float(), ctypes.c_int32()
    assert lib.gpt2_loss_scaler(None, 1.0, 2.0, 0.5, 10, 0) == L.GPT2_ERR_STATE
    assert lib.gpt2_loss_scaler_state(None, ctypes.byref(f), ctypes.byref(i), ctypes.byref(i)) == L.GPT2_ERR_ARG


def test_stream_probe_refuses_bad_arguments_before_any_launch(lib):
    # every case below is refused by the argument checks, before a HIP call
    assert lib.gpt2_stream_probe(3, None, None, 4, None) == L.GPT2_ERR_ARG            # no such mode
    assert lib.gpt2_stream_probe(0, None, ctypes.c_void_p(256), 4, None) == L.GPT2_ERR_ARG  # read without src
    assert lib.gpt2_stream_probe(1, None, None, 4, None) == L.GPT2_ERR_ARG            # write without dst
    assert lib.gpt2_stream_probe(2, ctypes.c_void_p(256), ctypes.c_void_p(264), 4, None) == L.GPT2_ERR_ARG  # misaligned
    assert lib.gpt2_stream_probe(1, None, ctypes.c_void_p(256), 6, None) == L.GPT2_ERR_ARG  # n % 4
    assert lib.gpt2_stream_probe(1, None, ctypes.c_void_p(256), 0, None) == L.GPT2_ERR_ARG  # empty
