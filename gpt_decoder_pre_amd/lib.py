"""ctypes binding of libgpt2.so (the C ABI in include/gpt2.h).

Argument marshalling only: every step of the training step runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
The library must be built (``python -m gpt_decoder_pre_amd.build``); there is
no fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from collections import OrderedDict

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libgpt2.so")

GPT2_OK = 0
GPT2_ERR_ARG = -1
GPT2_ERR_SEQ_TOO_LONG = -2
GPT2_ERR_BATCH = -3
GPT2_ERR_STATE = -4
GPT2_ERR_TOKEN = -5
GPT2_ERR_HIP = -6
GPT2_FP32 = 0
GPT2_BF16 = 1

ERROR_NAMES = {
    GPT2_ERR_ARG: "GPT2_ERR_ARG", GPT2_ERR_SEQ_TOO_LONG: "GPT2_ERR_SEQ_TOO_LONG",
    GPT2_ERR_BATCH: "GPT2_ERR_BATCH", GPT2_ERR_STATE: "GPT2_ERR_STATE",
    GPT2_ERR_TOKEN: "GPT2_ERR_TOKEN", GPT2_ERR_HIP: "GPT2_ERR_HIP",
}

# Every function the header declares.
EXPORTS = ("gpt2_init", "gpt2_forward_loss", "gpt2_backward", "gpt2_accumulate", "gpt2_clip_adamw_step",
           "gpt2_destroy", "gpt2_sync_status", "gpt2_sync_params", "gpt2_get_step", "gpt2_set_step",
           "gpt2_tensor_info", "gpt2_activation", "gpt2_timing_enable", "gpt2_timing_read")


class Gpt2Error(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {ERROR_NAMES.get(code, code)}")
        self.code = code


class gpt2_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("vocab_size", ctypes.c_int32),
                ("padded_vocab_size", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("max_batch", ctypes.c_int32)]


class gpt2_buffers(ctypes.Structure):
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("adam_m", ctypes.c_void_p),
                ("adam_v", ctypes.c_void_p), ("params_bf16", ctypes.c_void_p), ("workspace", ctypes.c_void_p)]


class gpt2_sizes(ctypes.Structure):
    _fields_ = [("n_params", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("params_bf16_bytes", ctypes.c_int64)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libgpt2.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gpt_decoder_pre_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    sig = {
        "gpt2_init": (I, [ctypes.POINTER(gpt2_config), ctypes.POINTER(gpt2_buffers), P,
                          ctypes.POINTER(gpt2_sizes), ctypes.POINTER(P)]),
        "gpt2_forward_loss": (I, [P, P, P, I, I, F, P]),
        "gpt2_backward": (I, [P]),
        "gpt2_accumulate": (I, [P, P, P, I, I, I, P]),
        "gpt2_clip_adamw_step": (I, [P, F, F, F, F, F, F, P, P]),
        "gpt2_destroy": (None, [P]),
        "gpt2_sync_status": (I, [P]),
        "gpt2_sync_params": (I, [P]),
        "gpt2_get_step": (I64, [P]),
        "gpt2_set_step": (I, [P, I64]),
        "gpt2_tensor_info": (I, [ctypes.POINTER(gpt2_config), I, ctypes.POINTER(ctypes.c_char_p),
                                 ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_int32),
                                 ctypes.POINTER(I64)]),
        "gpt2_activation": (I, [P, ctypes.c_char_p, I, ctypes.POINTER(P), ctypes.POINTER(I64),
                                ctypes.POINTER(ctypes.c_int32)]),
        "gpt2_timing_enable": (I, [P, ctypes.c_char_p]),
        "gpt2_timing_read": (I, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, what: str) -> None:
    if code != GPT2_OK:
        raise Gpt2Error(code, what)


def make_config(shape, precision: str, max_batch: int) -> gpt2_config:
    return gpt2_config(shape.n_layer, shape.n_head, shape.n_embd, shape.block_size, shape.vocab_size,
                       shape.padded_vocab_size, GPT2_BF16 if precision == "bf16" else GPT2_FP32, max_batch)


def query_sizes(cfg: gpt2_config) -> gpt2_sizes:
    lib = load_library()
    sz = gpt2_sizes()
    _check(lib.gpt2_init(ctypes.byref(cfg), None, None, ctypes.byref(sz), None), "gpt2_init (size query)")
    return sz


def tensor_layout(cfg: gpt2_config) -> "OrderedDict[str, tuple]":
    """name -> (offset, shape) of every parameter tensor, from the library."""
    lib = load_library()
    out = OrderedDict()
    i = 0
    while True:
        name = ctypes.c_char_p()
        off, numel = ctypes.c_int64(), ctypes.c_int64()
        nd = ctypes.c_int32()
        dims = (ctypes.c_int64 * 3)()
        if lib.gpt2_tensor_info(ctypes.byref(cfg), i, ctypes.byref(name), ctypes.byref(off), ctypes.byref(numel),
                                ctypes.byref(nd), dims) != GPT2_OK:
            break
        out[name.value.decode()] = (off.value, tuple(dims[k] for k in range(nd.value)))
        i += 1
    return out


class GPT2Step:
    """One context of the C ABI with its caller-owned device buffers (torch)."""

    def __init__(self, shape, precision: str = "bf16", max_batch: int = 1, device: str = "cuda"):
        import torch
        self.torch = torch
        self.lib = load_library()
        self.shape = shape
        self.precision = precision
        self.cfg = make_config(shape, precision, max_batch)
        self.sizes = query_sizes(self.cfg)
        self.layout = tensor_layout(self.cfg)
        n = self.sizes.n_params
        dev = torch.device(device)
        self.device = dev
        self.params = torch.zeros(n, dtype=torch.float32, device=dev)
        self.grads = torch.empty(n, dtype=torch.float32, device=dev)
        self.m = torch.empty(n, dtype=torch.float32, device=dev)
        self.v = torch.empty(n, dtype=torch.float32, device=dev)
        self.params_bf16 = (torch.empty(n, dtype=torch.bfloat16, device=dev) if precision == "bf16" else None)
        ws = self.sizes.workspace_bytes
        self.workspace = torch.empty(ws + 256, dtype=torch.uint8, device=dev)
        base = self.workspace.data_ptr()
        ws_ptr = (base + 255) // 256 * 256
        self.bufs = gpt2_buffers(self.params.data_ptr(), self.grads.data_ptr(), self.m.data_ptr(),
                                 self.v.data_ptr(),
                                 self.params_bf16.data_ptr() if self.params_bf16 is not None else None, ws_ptr)
        self.stream = torch.cuda.current_stream(dev)
        ctx = ctypes.c_void_p()
        _check(self.lib.gpt2_init(ctypes.byref(self.cfg), ctypes.byref(self.bufs),
                                  ctypes.c_void_p(self.stream.cuda_stream), None, ctypes.byref(ctx)), "gpt2_init")
        self.ctx = ctx
        self.d_loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.d_norm = torch.zeros(1, dtype=torch.float32, device=dev)
        self.d_clipped = torch.zeros(1, dtype=torch.int32, device=dev)

    # ---- marshalling of the flat parameter layout ----
    def _flat_view(self, flat, name):
        off, shp = self.layout[name]
        k = 1
        for d in shp:
            k *= d
        return flat[off:off + k].view(*shp)

    def load_params(self, params: dict) -> None:
        """Copy a dict of host arrays (canonical names) into the fp32 master
        weights and rebuild the bf16 copy."""
        torch = self.torch
        for name in self.layout:
            self._flat_view(self.params, name).copy_(torch.as_tensor(params[name]))
        _check(self.lib.gpt2_sync_params(self.ctx), "gpt2_sync_params")

    def load_state(self, name_to_m: dict, name_to_v: dict, step: int) -> None:
        torch = self.torch
        for name in self.layout:
            self._flat_view(self.m, name).copy_(torch.as_tensor(name_to_m[name], dtype=torch.float32))
            self._flat_view(self.v, name).copy_(torch.as_tensor(name_to_v[name], dtype=torch.float32))
        _check(self.lib.gpt2_set_step(self.ctx, step), "gpt2_set_step")

    def to_dict(self, flat) -> "OrderedDict[str, object]":
        return OrderedDict((n, self._flat_view(flat, n)) for n in self.layout)

    # ---- the C ABI ----
    def forward_loss(self, idx, targets, loss_scale: float = 1.0):
        B, T = idx.shape
        _check(self.lib.gpt2_forward_loss(self.ctx, ctypes.c_void_p(idx.data_ptr()),
                                          ctypes.c_void_p(targets.data_ptr()), B, T, loss_scale,
                                          ctypes.c_void_p(self.d_loss.data_ptr())), "gpt2_forward_loss")
        return self.d_loss

    def backward(self) -> None:
        _check(self.lib.gpt2_backward(self.ctx), "gpt2_backward")

    def accumulate(self, idx, targets):
        """idx, targets: int32 device tensors (k, B, T)."""
        k, B, T = idx.shape
        _check(self.lib.gpt2_accumulate(self.ctx, ctypes.c_void_p(idx.data_ptr()),
                                        ctypes.c_void_p(targets.data_ptr()), k, B, T,
                                        ctypes.c_void_p(self.d_loss.data_ptr())), "gpt2_accumulate")
        return self.d_loss

    def clip_adamw_step(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0):
        _check(self.lib.gpt2_clip_adamw_step(self.ctx, lr, beta1, beta2, eps, weight_decay, max_norm,
                                             ctypes.c_void_p(self.d_norm.data_ptr()),
                                             ctypes.c_void_p(self.d_clipped.data_ptr())), "gpt2_clip_adamw_step")
        return self.d_norm, self.d_clipped

    def sync_status(self) -> int:
        return self.lib.gpt2_sync_status(self.ctx)

    def step_count(self) -> int:
        return int(self.lib.gpt2_get_step(self.ctx))

    def activation(self, name: str, layer: int = 0):
        """A saved activation of the last forward as a torch view (no copy)."""
        torch = self.torch
        ptr, numel, dt = ctypes.c_void_p(), ctypes.c_int64(), ctypes.c_int32()
        _check(self.lib.gpt2_activation(self.ctx, name.encode(), layer, ctypes.byref(ptr), ctypes.byref(numel),
                                        ctypes.byref(dt)), f"gpt2_activation({name})")
        dtype = {0: torch.float32, 1: torch.bfloat16, 2: torch.int32}[dt.value]
        esz = {0: 4, 1: 2, 2: 4}[dt.value]
        base = self.workspace.data_ptr()
        off = ptr.value - base
        raw = self.workspace[off:off + numel.value * esz]
        return raw.view(dtype)

    def timing_enable(self, site) -> None:
        _check(self.lib.gpt2_timing_enable(self.ctx, site.encode() if site is not None else None),
               "gpt2_timing_enable")

    def timing_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        fl, by = ctypes.c_double(), ctypes.c_double()
        _check(self.lib.gpt2_timing_read(self.ctx, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl),
                                         ctypes.byref(by)), "gpt2_timing_read")
        return ms.value, n.value, fl.value, by.value

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self.lib.gpt2_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
