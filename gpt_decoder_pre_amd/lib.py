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
GPT2_ERR_IO = -7
GPT2_FP32 = 0
GPT2_BF16 = 1
GPT2_FP16 = 2
PRECISIONS = {"fp32": GPT2_FP32, "bf16": GPT2_BF16, "fp16": GPT2_FP16}
GPT2_UNTIED_HEAD = 1
GPT2_NO_QKV_BIAS = 2

ERROR_NAMES = {
    GPT2_ERR_ARG: "GPT2_ERR_ARG", GPT2_ERR_SEQ_TOO_LONG: "GPT2_ERR_SEQ_TOO_LONG",
    GPT2_ERR_BATCH: "GPT2_ERR_BATCH", GPT2_ERR_STATE: "GPT2_ERR_STATE",
    GPT2_ERR_TOKEN: "GPT2_ERR_TOKEN", GPT2_ERR_HIP: "GPT2_ERR_HIP", GPT2_ERR_IO: "GPT2_ERR_IO",
}

# Every function the header declares.
EXPORTS = ("gpt2_init", "gpt2_forward_loss", "gpt2_backward", "gpt2_accumulate", "gpt2_clip_adamw_step",
           "gpt2_destroy", "gpt2_sync_status", "gpt2_sync_params", "gpt2_get_step", "gpt2_set_step",
           "gpt2_tensor_info", "gpt2_activation", "gpt2_timing_enable", "gpt2_timing_read", "gpt2_timing_site",
           "gpt2_embedding_backward", "gpt2_clip_adamw_step_static", "gpt2_loss_scaler", "gpt2_loss_scaler_state",
           "gpt2_lr_at", "gpt2_loader_open", "gpt2_loader_next", "gpt2_loader_next_host", "gpt2_loader_state",
           "gpt2_loader_seek", "gpt2_loader_close", "gpt2_checkpoint_save", "gpt2_checkpoint_load",
           "gpt2_infer_init", "gpt2_infer_prefill", "gpt2_infer_decode", "gpt2_infer_length", "gpt2_sample",
           "gpt2_infer_sync_status", "gpt2_infer_destroy", "gpt2_stream_probe")


class Gpt2Error(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {ERROR_NAMES.get(code, code)}")
        self.code = code


class gpt2_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("vocab_size", ctypes.c_int32),
                ("padded_vocab_size", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("variant", ctypes.c_int32)]


class gpt2_buffers(ctypes.Structure):
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("adam_m", ctypes.c_void_p),
                ("adam_v", ctypes.c_void_p), ("params_bf16", ctypes.c_void_p), ("workspace", ctypes.c_void_p)]


class gpt2_lr_schedule(ctypes.Structure):
    _fields_ = [("max_lr", ctypes.c_double), ("min_lr", ctypes.c_double), ("warmup_steps", ctypes.c_int64),
                ("max_steps", ctypes.c_int64)]


class gpt2_infer_sizes(ctypes.Structure):
    _fields_ = [("cache_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


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
        "gpt2_embedding_backward": (I, [P, P, P, I, I]),
        "gpt2_lr_at": (ctypes.c_double, [ctypes.POINTER(gpt2_lr_schedule), I64]),
        "gpt2_loader_open": (I, [ctypes.POINTER(ctypes.c_char_p), I, ctypes.c_int32, ctypes.c_int32, I, I, I,
                                 ctypes.POINTER(P)]),
        "gpt2_loader_next": (I, [P, P, P, P]),
        "gpt2_loader_next_host": (I, [P, P, P]),
        "gpt2_loader_state": (I, [P, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "gpt2_loader_seek": (I, [P, I64, I64]),
        "gpt2_loader_close": (None, [P]),
        "gpt2_checkpoint_save": (I, [P, ctypes.c_char_p, ctypes.POINTER(I64), I]),
        "gpt2_checkpoint_load": (I, [P, ctypes.c_char_p, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_int)]),
        "gpt2_clip_adamw_step_static": (I, [ctypes.POINTER(gpt2_config), ctypes.POINTER(gpt2_buffers), P, I64,
                                            F, F, F, F, F, F, P, P]),
        "gpt2_loss_scaler": (I, [P, F, F, F, ctypes.c_int32, ctypes.c_int32]),
        "gpt2_loss_scaler_state": (I, [P, ctypes.POINTER(F), ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32)]),
        "gpt2_infer_init": (I, [ctypes.POINTER(gpt2_config), P, P, P, P, P, ctypes.POINTER(gpt2_infer_sizes),
                                ctypes.POINTER(P)]),
        "gpt2_infer_prefill": (I, [P, P, I, I, P]),
        "gpt2_infer_decode": (I, [P, P, P]),
        "gpt2_infer_length": (I, [P]),
        "gpt2_sample": (I, [P, I64, I, I, F, I, F, P, P, P]),
        "gpt2_infer_sync_status": (I, [P]),
        "gpt2_infer_destroy": (None, [P]),
        "gpt2_stream_probe": (I, [I, P, P, I64, P]),
        "gpt2_timing_site": (I, [P, I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
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
    variant = (0 if getattr(shape, "tied", True) else GPT2_UNTIED_HEAD) | \
              (0 if getattr(shape, "qkv_bias", True) else GPT2_NO_QKV_BIAS)
    return gpt2_config(shape.n_layer, shape.n_head, shape.n_embd, shape.block_size, shape.vocab_size,
                       shape.padded_vocab_size, PRECISIONS[precision], max_batch, variant)


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
        # the 16-bit copy of the weights (bf16, or fp16 in the fp16 mode)
        h16 = {"bf16": torch.bfloat16, "fp16": torch.float16}.get(precision)
        self.params_bf16 = torch.empty(n, dtype=h16, device=dev) if h16 is not None else None
        ws = self.sizes.workspace_bytes
        self.workspace = torch.empty(ws + 256, dtype=torch.uint8, device=dev)
        base = self.workspace.data_ptr()
        ws_ptr = (base + 255) // 256 * 256
        self.bufs = gpt2_buffers(self.params.data_ptr(), self.grads.data_ptr(), self.m.data_ptr(),
                                 self.v.data_ptr(),
                                 self.params_bf16.data_ptr() if self.params_bf16 is not None else None, ws_ptr)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
            self.device = dev
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
    def _check_tokens(self, idx, targets, ndim: int, what: str) -> None:
        """The C ABI reads int32 (.., T) row-major device arrays: anything else
        (torch's default int64 ids, a strided view, host memory) would be read
        as different tokens, so it is refused here."""
        torch = self.torch
        for name, t in (("idx", idx), ("targets", targets)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{what}: {name} must be a torch tensor")
            if t.dtype != torch.int32:
                raise TypeError(f"{what}: {name} must be int32, got {t.dtype}")
            if t.dim() != ndim:
                raise ValueError(f"{what}: {name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
            if not t.is_contiguous():
                raise ValueError(f"{what}: {name} must be contiguous")
            if t.device != self.device:
                raise ValueError(f"{what}: {name} is on {t.device}, the context is on {self.device}")
        if idx.shape != targets.shape:
            raise ValueError(f"{what}: idx {tuple(idx.shape)} and targets {tuple(targets.shape)} differ in shape")

    def forward_loss(self, idx, targets, loss_scale: float = 1.0):
        self._check_tokens(idx, targets, 2, "forward_loss")
        B, T = idx.shape
        _check(self.lib.gpt2_forward_loss(self.ctx, ctypes.c_void_p(idx.data_ptr()),
                                          ctypes.c_void_p(targets.data_ptr()), B, T, loss_scale,
                                          ctypes.c_void_p(self.d_loss.data_ptr())), "gpt2_forward_loss")
        return self.d_loss

    def backward(self) -> None:
        _check(self.lib.gpt2_backward(self.ctx), "gpt2_backward")

    def accumulate(self, idx, targets):
        """idx, targets: int32 device tensors (k, B, T)."""
        self._check_tokens(idx, targets, 3, "accumulate")
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

    def embedding_backward(self, idx, dx0) -> None:
        """idx: int32 (B, T), dx0: fp32 (B, T, C) device tensors; adds the
        embedding gradient of dx0 into grads (wte and wpe)."""
        torch = self.torch
        self._check_tokens(idx, idx, 2, "embedding_backward")
        B, T = idx.shape
        if dx0.dtype != torch.float32 or not dx0.is_contiguous() or dx0.device != self.device or \
                tuple(dx0.shape) != (B, T, self.shape.n_embd):
            raise ValueError("embedding_backward: dx0 must be a contiguous fp32 (B, T, C) tensor on the device")
        _check(self.lib.gpt2_embedding_backward(self.ctx, ctypes.c_void_p(idx.data_ptr()),
                                                ctypes.c_void_p(dx0.data_ptr()), B, T), "gpt2_embedding_backward")

    def clip_adamw_step_static(self, t, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0):
        """gpt2_clip_adamw_step_static on this object's buffers at step t (the
        context's own step counter is not used or changed)."""
        _check(self.lib.gpt2_clip_adamw_step_static(ctypes.byref(self.cfg), ctypes.byref(self.bufs),
                                                    ctypes.c_void_p(self.stream.cuda_stream), t, lr, beta1, beta2,
                                                    eps, weight_decay, max_norm,
                                                    ctypes.c_void_p(self.d_norm.data_ptr()),
                                                    ctypes.c_void_p(self.d_clipped.data_ptr())),
               "gpt2_clip_adamw_step_static")
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
        dtype = {0: torch.float32, 1: torch.bfloat16, 2: torch.int32, 3: torch.float16}[dt.value]
        esz = {0: 4, 1: 2, 2: 4, 3: 2}[dt.value]
        base = self.workspace.data_ptr()
        off = ptr.value - base
        raw = self.workspace[off:off + numel.value * esz]
        return raw.view(dtype)

    def loss_scaler(self, scale: float, growth_factor: float = 2.0, backoff_factor: float = 0.5,
                    growth_interval: int = 2000, good_steps: int = 0) -> None:
        """Sets the dynamic loss scaler of an fp16 context."""
        _check(self.lib.gpt2_loss_scaler(self.ctx, scale, growth_factor, backoff_factor, growth_interval, good_steps),
               "gpt2_loss_scaler")

    def loss_scaler_state(self):
        """(scale, good_steps, skipped) of an fp16 context's loss scaler."""
        sc, good, sk = ctypes.c_float(), ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib.gpt2_loss_scaler_state(self.ctx, ctypes.byref(sc), ctypes.byref(good), ctypes.byref(sk)),
               "gpt2_loss_scaler_state")
        return sc.value, good.value, sk.value

    def timing_enable(self, site) -> None:
        _check(self.lib.gpt2_timing_enable(self.ctx, site.encode() if site is not None else None),
               "gpt2_timing_enable")

    def timing_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        fl, by = ctypes.c_double(), ctypes.c_double()
        _check(self.lib.gpt2_timing_read(self.ctx, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl),
                                         ctypes.byref(by)), "gpt2_timing_read")
        return ms.value, n.value, fl.value, by.value

    def timing_sites(self):
        """Per-site totals of the recorded launches: list of dicts with the
        site name, summed ms, launch count, flops, bytes and the GEMM tile
        configuration of its last launch."""
        out = []
        i = 0
        while True:
            name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
            fl, by, cfg = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
            code = self.lib.gpt2_timing_site(self.ctx, i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n),
                                             ctypes.byref(fl), ctypes.byref(by), ctypes.byref(cfg))
            if code == GPT2_ERR_ARG:
                break
            _check(code, "gpt2_timing_site")
            out.append({"site": name.value.decode(), "ms": ms.value, "launches": n.value, "flops": fl.value,
                        "bytes": by.value, "gemm_cfg": cfg.value})
            i += 1
        return out

    def checkpoint_save(self, path: str, extra=()) -> None:
        """Training state (params, AdamW moments, step counter, extra int64
        words such as the loader position) to a file."""
        ex = (ctypes.c_int64 * 16)(*extra)
        _check(self.lib.gpt2_checkpoint_save(self.ctx, os.fsencode(path), ex, len(extra)), "gpt2_checkpoint_save")

    def checkpoint_load(self, path: str):
        """Restores a checkpoint; returns its extra words."""
        ex = (ctypes.c_int64 * 16)()
        n = ctypes.c_int(16)
        _check(self.lib.gpt2_checkpoint_load(self.ctx, os.fsencode(path), ex, ctypes.byref(n)),
               "gpt2_checkpoint_load")
        return tuple(ex[i] for i in range(n.value))

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self.lib.gpt2_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lr_at(max_lr: float, min_lr: float, warmup_steps: int, max_steps: int, step: int) -> float:
    """The library's warmup + cosine learning rate for optimizer step `step`."""
    lib = load_library()
    sched = gpt2_lr_schedule(max_lr, min_lr, warmup_steps, max_steps)
    return float(lib.gpt2_lr_at(ctypes.byref(sched), step))


class TokenLoader:
    """The library's sequential loader over token shard files (uint16 or
    int32 ids): one call of next() gives one optimizer step of k micro-batches
    of B x T tokens."""

    def __init__(self, paths, vocab_size: int, k: int, B: int, T: int, dtype: str = "uint16"):
        self.lib = load_library()
        self.shape = (k, B, T)
        arr = (ctypes.c_char_p * len(paths))(*[os.fsencode(p) for p in paths])
        ld = ctypes.c_void_p()
        _check(self.lib.gpt2_loader_open(arr, len(paths), 0 if dtype == "uint16" else 1, vocab_size, k, B, T,
                                         ctypes.byref(ld)), "gpt2_loader_open")
        self.ld = ld

    def next_host(self):
        import numpy as np
        k, B, T = self.shape
        x = np.empty((k, B, T), np.int32)
        y = np.empty((k, B, T), np.int32)
        _check(self.lib.gpt2_loader_next_host(self.ld, x.ctypes.data_as(ctypes.c_void_p),
                                              y.ctypes.data_as(ctypes.c_void_p)), "gpt2_loader_next_host")
        return x, y

    def next_device(self, x, y, stream) -> None:
        """Fills the int32 (k, B, T) device tensors x, y on `stream`."""
        import torch
        for t in (x, y):
            if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != self.shape or not t.is_cuda:
                raise ValueError("next_device: x and y must be contiguous int32 (k, B, T) device tensors")
        _check(self.lib.gpt2_loader_next(self.ld, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                         ctypes.c_void_p(stream.cuda_stream)), "gpt2_loader_next")

    def state(self):
        sh, pos = ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib.gpt2_loader_state(self.ld, ctypes.byref(sh), ctypes.byref(pos)), "gpt2_loader_state")
        return sh.value, pos.value

    def seek(self, shard: int, pos: int) -> None:
        _check(self.lib.gpt2_loader_seek(self.ld, shard, pos), "gpt2_loader_seek")

    def close(self) -> None:
        if getattr(self, "ld", None):
            self.lib.gpt2_loader_close(self.ld)
            self.ld = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Decoder:
    """A decoding context of the C ABI (gpt2_infer.h) over the parameters of
    a GPT2Step (read, not copied): prefill, one-token steps and sampling."""

    def __init__(self, step: "GPT2Step", max_batch: int):
        import torch
        self.torch = torch
        self.lib = load_library()
        self.step = step
        cfg = make_config(step.shape, step.precision, max_batch)
        self.cfg = cfg
        sz = gpt2_infer_sizes()
        _check(self.lib.gpt2_infer_init(ctypes.byref(cfg), None, None, None, None, None, ctypes.byref(sz), None),
               "gpt2_infer_init (size query)")
        dev = step.device
        self.cache = torch.empty(sz.cache_bytes + 256, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(sz.workspace_bytes + 256, dtype=torch.uint8, device=dev)
        al = lambda t: (t.data_ptr() + 255) // 256 * 256  # noqa: E731
        self.stream = step.stream
        ctx = ctypes.c_void_p()
        _check(self.lib.gpt2_infer_init(ctypes.byref(cfg), ctypes.c_void_p(step.params.data_ptr()),
                                        ctypes.c_void_p(step.params_bf16.data_ptr()) if step.params_bf16 is not None
                                        else None, ctypes.c_void_p(al(self.cache)), ctypes.c_void_p(al(self.ws)),
                                        ctypes.c_void_p(self.stream.cuda_stream), None, ctypes.byref(ctx)),
               "gpt2_infer_init")
        self.ctx = ctx
        self.vp = step.shape.padded_vocab_size
        self.B = 0

    def _logits(self, B):
        return self.torch.empty((B, self.vp), dtype=self.torch.float32, device=self.step.device)

    def prefill(self, idx):
        """idx: int32 (B, T) device tensor; returns fp32 (B, Vp) logits of the last position."""
        torch = self.torch
        if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous() or idx.device != self.step.device:
            raise ValueError("prefill: idx must be a contiguous int32 (B, T) tensor on the device")
        B, T = idx.shape
        out = self._logits(B)
        _check(self.lib.gpt2_infer_prefill(self.ctx, ctypes.c_void_p(idx.data_ptr()), B, T,
                                           ctypes.c_void_p(out.data_ptr())), "gpt2_infer_prefill")
        self.B = B
        return out

    def decode(self, tokens):
        """tokens: int32 (B,) device tensor; returns fp32 (B, Vp) logits."""
        torch = self.torch
        if tokens.dtype != torch.int32 or tuple(tokens.shape) != (self.B,) or not tokens.is_contiguous() \
                or tokens.device != self.step.device:
            raise ValueError("decode: tokens must be a contiguous int32 (B,) tensor on the device")
        out = self._logits(self.B)
        _check(self.lib.gpt2_infer_decode(self.ctx, ctypes.c_void_p(tokens.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr())), "gpt2_infer_decode")
        return out

    def length(self) -> int:
        return int(self.lib.gpt2_infer_length(self.ctx))

    def sample(self, logits, uniform, temperature=1.0, top_k=0, top_p=1.0):
        return sample(logits, uniform, self.step.shape.vocab_size, temperature, top_k, top_p, self.stream)

    def sync_status(self) -> int:
        return self.lib.gpt2_infer_sync_status(self.ctx)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self.lib.gpt2_infer_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sample(logits, uniform, vocab_size, temperature=1.0, top_k=0, top_p=1.0, stream=None):
    """gpt2_sample: logits fp32 (B, ld) and uniform fp32 (B,) device tensors;
    returns int32 (B,) tokens."""
    import torch
    lib = load_library()
    B, ld = logits.shape
    if logits.dtype != torch.float32 or not logits.is_contiguous() or uniform.dtype != torch.float32 \
            or tuple(uniform.shape) != (B,) or not uniform.is_contiguous():
        raise ValueError("sample: logits fp32 (B, ld) and uniform fp32 (B,) contiguous device tensors")
    out = torch.empty(B, dtype=torch.int32, device=logits.device)
    st = stream if stream is not None else torch.cuda.current_stream(logits.device)
    _check(lib.gpt2_sample(ctypes.c_void_p(logits.data_ptr()), ld, B, vocab_size, temperature, top_k, top_p,
                           ctypes.c_void_p(uniform.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                           ctypes.c_void_p(st.cuda_stream)), "gpt2_sample")
    return out


# gpt2_stream_probe modes
PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2


def probe_partials(n: int) -> int:
    """Floats the read probe writes for n input floats (one per wave of 64
    threads, eight 16-byte loads each)."""
    return 4 * ((n + 8191) // 8192)


def stream_probe(mode, src, dst, stream=None):
    """gpt2_stream_probe: one launch of a plain HBM stream over fp32 device
    tensors (src unused for PROBE_WRITE; for PROBE_READ, dst receives the
    per-wave partial sums and must hold probe_partials(n) floats)."""
    import torch
    lib = load_library()
    if mode not in (PROBE_READ, PROBE_WRITE, PROBE_COPY) or dst is None or (mode != PROBE_WRITE and src is None):
        raise ValueError("stream_probe: mode PROBE_READ / PROBE_WRITE / PROBE_COPY, dst, and src unless writing")
    n = (src if mode != PROBE_WRITE else dst).numel()
    for t in (src, dst):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("stream_probe: contiguous fp32 device tensors")
    if mode == PROBE_READ and dst.numel() < probe_partials(n):
        raise ValueError(f"stream_probe: the read probe writes {probe_partials(n)} partial sums")
    if mode == PROBE_COPY and dst.numel() < n:
        raise ValueError("stream_probe: dst smaller than src")
    dev = dst.device
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    _check(lib.gpt2_stream_probe(mode, ctypes.c_void_p(src.data_ptr() if src is not None else 0),
                                 ctypes.c_void_p(dst.data_ptr()), n, ctypes.c_void_p(st.cuda_stream)),
           "gpt2_stream_probe")
