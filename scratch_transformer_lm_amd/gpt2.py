"""Thin ctypes binding of libgpt2_mi355x.so (include/gpt2.h).

Argument marshalling only: torch provides device memory and the current HIP stream,
every step of the computation runs in the library's kernels.  There is no fallback: if
the library is missing this module raises.
"""
from __future__ import annotations

import ctypes as ct
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gpt2.h")

GPT2_OK, GPT2_EINVAL, GPT2_ESTATE, GPT2_EDEVICE, GPT2_ENOMEM, GPT2_ESCRATCH = 0, -1, -2, -3, -4, -5
PARAM_NAMES = ("wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb")
ACT_NAMES = ("encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "att_lse", "residual2",
             "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "residual3", "lnf", "lnf_mean",
             "lnf_rstd", "logits", "logits_lse", "losses")


class Config(ct.Structure):
    _fields_ = [("max_seq_len", ct.c_int), ("vocab_size", ct.c_int), ("num_layers", ct.c_int),
                ("num_heads", ct.c_int), ("channels", ct.c_int)]


class Buffers(ct.Structure):
    _fields_ = [(n, ct.c_void_p) for n in ("params", "grads", "m", "v", "acts", "grad_scratch")]


class GPT2Error(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_LIB = None


def header_functions() -> list[str]:
    """Names of the functions include/gpt2.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(gpt2_[a-z_0-9]+)\s*\(", text)


def load() -> ct.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run scratch_transformer_lm_amd/build.py "
                           "(there is no CPU fallback)")
    lib = ct.CDLL(LIB_PATH)
    P, sz, i, f = ct.c_void_p, ct.c_size_t, ct.c_int, ct.c_float
    C = ct.POINTER(Config)
    lib.gpt2_num_parameters.argtypes = [C]
    lib.gpt2_num_parameters.restype = sz
    lib.gpt2_param_layout.argtypes = [C, P, P]
    lib.gpt2_param_layout.restype = i
    lib.gpt2_arena_sizes.argtypes = [C, i, i, ct.POINTER(sz), ct.POINTER(sz)]
    lib.gpt2_arena_sizes.restype = i
    lib.gpt2_arena_sizes_variant.argtypes = [C, i, i, i, ct.POINTER(sz), ct.POINTER(sz)]
    lib.gpt2_arena_sizes_variant.restype = i
    lib.gpt2_build.argtypes = [ct.POINTER(P), C, i, i, ct.POINTER(Buffers), P]
    lib.gpt2_build.restype = i
    lib.gpt2_build_variant.argtypes = [ct.POINTER(P), C, i, i, ct.POINTER(Buffers), P, i]
    lib.gpt2_build_variant.restype = i
    lib.gpt2_forward.argtypes = [P, P, P, i, i]
    lib.gpt2_forward.restype = f
    lib.gpt2_zero_grad.argtypes = [P]
    lib.gpt2_zero_grad.restype = i
    lib.gpt2_backward.argtypes = [P]
    lib.gpt2_backward.restype = i
    lib.gpt2_update.argtypes = [P, f, f, f, f, f, i]
    lib.gpt2_update.restype = i
    lib.gpt2_last_error.argtypes = [P]
    lib.gpt2_last_error.restype = i
    lib.gpt2_strerror.argtypes = [i]
    lib.gpt2_strerror.restype = ct.c_char_p
    lib.gpt2_free.argtypes = [P]
    lib.gpt2_free.restype = None
    lib.gpt2_activation_view.argtypes = [P, i, i] + [ct.POINTER(sz)] * 4
    lib.gpt2_activation_view.restype = i
    lib.gpt2_profile_enable.argtypes = [P, i]
    lib.gpt2_profile_enable.restype = i
    lib.gpt2_profile_filter.argtypes = [P, ct.c_char_p]
    lib.gpt2_profile_filter.restype = i
    lib.gpt2_profile_collect.argtypes = [P]
    lib.gpt2_profile_collect.restype = i
    lib.gpt2_profile_entry.argtypes = [P, i, ct.POINTER(ct.c_char_p), ct.POINTER(ct.c_long),
                                       ct.POINTER(ct.c_double), ct.POINTER(ct.c_double),
                                       ct.POINTER(ct.c_double)]
    lib.gpt2_profile_entry.restype = i
    lib.gpt2_backward_update.argtypes = [P, f, f, f, f, f, i]
    lib.gpt2_backward_update.restype = i
    lib.gpt2_sample.argtypes = [P, P, P, i, P]
    lib.gpt2_sample.restype = i
    lib.gpt2_generate.argtypes = [P, P, i, i, P]
    lib.gpt2_generate.restype = i
    lib.gpt2_set_backward_streams.argtypes = [P, i]
    lib.gpt2_set_backward_streams.restype = i
    lib.gpt2_set_gemm_tiles.argtypes = [i]
    lib.gpt2_set_gemm_tiles.restype = i
    lib.gpt2_layernorm_forward.argtypes = [P, P, P, P, P, P, i, i, f, P]
    lib.gpt2_layernorm_forward.restype = i
    lib.gpt2_layernorm_backward_workspace.argtypes = [i, i]
    lib.gpt2_layernorm_backward_workspace.restype = sz
    lib.gpt2_layernorm_backward.argtypes = [P, P, P, P, P, P, P, P, i, i, P, sz, P]
    lib.gpt2_layernorm_backward.restype = i
    lib.gpt2_probe_mfma_out_floats.argtypes = []
    lib.gpt2_probe_mfma_out_floats.restype = sz
    lib.gpt2_probe_mfma.argtypes = [i, i, i, P, ct.POINTER(ct.c_double), P]
    lib.gpt2_probe_mfma.restype = i
    lib.gpt2_probe_copy.argtypes = [P, P, sz, i, P]
    lib.gpt2_probe_copy.restype = i
    lib.gpt2_layernorm_backward_noalloc_max_floats.argtypes = []
    lib.gpt2_layernorm_backward_noalloc_max_floats.restype = sz
    lib.gpt2_layernorm_backward_noalloc.argtypes = [P, P, P, P, P, P, P, P, i, i, P]
    lib.gpt2_layernorm_backward_noalloc.restype = i
    _LIB = lib
    return lib


def strerror(code: int) -> str:
    return load().gpt2_strerror(code).decode()


def config(shape) -> Config:
    return Config(shape.max_seq_len, shape.vocab_size, shape.num_layers, shape.num_heads,
                  shape.channels)


def num_parameters(shape) -> int:
    c = config(shape)
    return load().gpt2_num_parameters(ct.byref(c))


def param_layout(shape):
    c = config(shape)
    off = np.zeros(16, np.uint64)
    ln = np.zeros(16, np.uint64)
    rc = load().gpt2_param_layout(ct.byref(c), off.ctypes.data, ln.ctypes.data)
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_param_layout")
    return [int(x) for x in off], [int(x) for x in ln]


def arena_sizes(shape, B: int, T: int, variant: int = 0):
    c = config(shape)
    a, s = ct.c_size_t(), ct.c_size_t()
    rc = load().gpt2_arena_sizes_variant(ct.byref(c), B, T, variant, ct.byref(a), ct.byref(s))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_arena_sizes_variant")
    return a.value, s.value


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class GPT2:
    """One model: six torch device buffers and the library handle built over them."""

    def __init__(self, shape, B: int, T: int, device="cuda", stream=None, variant: int = 0):
        import torch
        self.lib = load()
        self.shape = shape
        self.B, self.T = B, T
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        n = num_parameters(shape)
        if n == 0:
            raise GPT2Error(GPT2_EINVAL, "gpt2_num_parameters")
        na, ns = arena_sizes(shape, B, T, variant)
        f32 = torch.float32
        self.params = torch.empty(n, dtype=f32, device=self.device)
        self.grads = torch.empty(n, dtype=f32, device=self.device)
        self.m = torch.empty(n, dtype=f32, device=self.device)
        self.v = torch.empty(n, dtype=f32, device=self.device)
        self.acts = torch.empty(na, dtype=f32, device=self.device)
        self.grad_scratch = torch.empty(ns, dtype=f32, device=self.device)
        self.offsets, self.lengths = param_layout(shape)
        bufs = Buffers(*(t.data_ptr() for t in (self.params, self.grads, self.m, self.v, self.acts,
                                                  self.grad_scratch)))
        h = ct.c_void_p()
        cfg = config(shape)
        rc = self.lib.gpt2_build_variant(ct.byref(h), ct.byref(cfg), B, T, ct.byref(bufs),
                                         _stream_ptr(self.stream), variant)
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_build_variant")
        self.variant = variant
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.gpt2_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the five calls -------------------------------------------------------------
    def forward(self, inputs, targets=None) -> float:
        """inputs/targets: int32 device tensors (B, T)."""
        B, T = inputs.shape
        tp = targets.data_ptr() if targets is not None else None
        return self.lib.gpt2_forward(self.h, inputs.data_ptr(), tp, B, T)

    def zero_grad(self) -> int:
        return self.lib.gpt2_zero_grad(self.h)

    def backward(self) -> int:
        return self.lib.gpt2_backward(self.h)

    def update(self, lr, beta1, beta2, eps, weight_decay, t) -> int:
        return self.lib.gpt2_update(self.h, lr, beta1, beta2, eps, weight_decay, t)

    def backward_update(self, lr, beta1, beta2, eps, weight_decay, t) -> int:
        return self.lib.gpt2_backward_update(self.h, lr, beta1, beta2, eps, weight_decay, t)

    def last_error(self) -> int:
        return self.lib.gpt2_last_error(self.h)

    def sample(self, rows, coins) -> np.ndarray:
        """gpt2_sample: next tokens at logits rows `rows` of the last forward for `coins` in [0,1)."""
        r = np.ascontiguousarray(rows, dtype=np.int32)
        c = np.ascontiguousarray(coins, dtype=np.float32)
        assert r.shape == c.shape and r.ndim == 1
        out = np.zeros(r.shape, dtype=np.int32)
        rc = self.lib.gpt2_sample(self.h, r.ctypes.data, c.ctypes.data, len(r), out.ctypes.data)
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_sample")
        return out

    def generate(self, prompt, total_len: int, coins) -> np.ndarray:
        """gpt2_generate: extends `prompt` to `total_len` tokens, one coin per new token."""
        p = np.ascontiguousarray(prompt, dtype=np.int32).reshape(-1)
        c = np.ascontiguousarray(coins, dtype=np.float32).reshape(-1)
        assert len(c) >= total_len - len(p)
        toks = np.zeros(total_len, dtype=np.int32)
        toks[:len(p)] = p
        rc = self.lib.gpt2_generate(self.h, toks.ctypes.data, len(p), total_len, c.ctypes.data)
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_generate")
        return toks

    def set_backward_streams(self, streams: int) -> None:
        """gpt2_set_backward_streams: 2 overlaps the weight gradients with the main chain."""
        rc = self.lib.gpt2_set_backward_streams(self.h, streams)
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_set_backward_streams")

    # -- per-kernel timing ------------------------------------------------------------
    def profile_enable(self, on: bool = True) -> bool:
        rc = self.lib.gpt2_profile_enable(self.h, int(on))
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_profile_enable")
        return True

    def profile_filter(self, kernel_name: str | None) -> None:
        rc = self.lib.gpt2_profile_filter(self.h, kernel_name.encode() if kernel_name else None)
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_profile_filter")

    def profile_entries(self) -> list[dict]:
        n = self.lib.gpt2_profile_collect(self.h)
        if n < 0:
            raise GPT2Error(n, "gpt2_profile_collect")
        out = []
        for i in range(n):
            name, cnt = ct.c_char_p(), ct.c_long()
            ms, fl, by = ct.c_double(), ct.c_double(), ct.c_double()
            rc = self.lib.gpt2_profile_entry(self.h, i, ct.byref(name), ct.byref(cnt), ct.byref(ms),
                                             ct.byref(fl), ct.byref(by))
            if rc != GPT2_OK:
                raise GPT2Error(rc, "gpt2_profile_entry")
            out.append(dict(name=name.value.decode(), launches=cnt.value, ms=ms.value,
                            flops=fl.value, bytes=by.value))
        return out

    # -- views ------------------------------------------------------------------------
    def tensor(self, buf, name: str):
        i = PARAM_NAMES.index(name)
        return buf[self.offsets[i]: self.offsets[i] + self.lengths[i]]

    def activation(self, name: str, layer: int = 0):
        """(rows, cols) view of an activation tensor (padding columns dropped)."""
        vals = [ct.c_size_t() for _ in range(4)]
        rc = self.lib.gpt2_activation_view(self.h, ACT_NAMES.index(name), layer,
                                           *[ct.byref(v) for v in vals])
        if rc != GPT2_OK:
            raise GPT2Error(rc, "gpt2_activation_view")
        off, rows, cols, ld = (v.value for v in vals)
        return self.acts[off: off + rows * ld].view(rows, ld)[:, :cols]


GEMM_TILES_AUTO, GEMM_TILES_128, GEMM_TILES_96 = 0, 1, 2
# gpt2_build_variant bits: Llama-style layers (RMSNorm, rotary positions), mixed precision
VARIANT_RMSNORM, VARIANT_ROPE, VARIANT_BF16 = 1, 2, 4


def set_gemm_tiles(policy: int) -> None:
    """gpt2_set_gemm_tiles: tile width of the forward and dgrad matmuls (process-wide)."""
    rc = load().gpt2_set_gemm_tiles(policy)
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_set_gemm_tiles")


def layernorm_forward(y, mean, rstd, x, w, b, eps=1e-5, stream=None) -> None:
    N, C = x.shape
    rc = load().gpt2_layernorm_forward(y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), x.data_ptr(),
                                       w.data_ptr(), b.data_ptr(), N, C, eps, _stream_ptr(stream))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_layernorm_forward")


def layernorm_backward_workspace(N: int, C: int) -> int:
    return load().gpt2_layernorm_backward_workspace(N, C)


def layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, workspace, stream=None) -> None:
    N, C = x.shape
    rc = load().gpt2_layernorm_backward(dx.data_ptr(), dw.data_ptr(), db.data_ptr(), dy.data_ptr(),
                                        x.data_ptr(), w.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                        N, C, workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_layernorm_backward")


def layernorm_backward_noalloc_max_floats() -> int:
    return load().gpt2_layernorm_backward_noalloc_max_floats()


def layernorm_backward_noalloc(dx, dw, db, dy, x, w, mean, rstd, stream=None) -> None:
    """gpt2_layernorm_backward_noalloc: as layernorm_backward, with the library's fixed
    device scratch instead of a workspace."""
    N, C = x.shape
    rc = load().gpt2_layernorm_backward_noalloc(dx.data_ptr(), dw.data_ptr(), db.data_ptr(), dy.data_ptr(),
                                                x.data_ptr(), w.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                                N, C, _stream_ptr(stream))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_layernorm_backward_noalloc")


def probe_mfma_out_floats() -> int:
    return load().gpt2_probe_mfma_out_floats()


def probe_mfma(kind: int, iters: int, out, blocks: int = 1024, stream=None) -> float:
    """gpt2_probe_mfma: enqueue one matrix-core probe launch; returns the flops it executes."""
    fl = ct.c_double()
    rc = load().gpt2_probe_mfma(kind, iters, blocks, out.data_ptr(), ct.byref(fl), _stream_ptr(stream))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_probe_mfma")
    return fl.value


def probe_copy(dst, src, blocks: int = 2048, stream=None) -> None:
    """gpt2_probe_copy: dst[:] = src[:] (float32 device tensors of equal size)."""
    assert dst.numel() == src.numel()
    rc = load().gpt2_probe_copy(dst.data_ptr(), src.data_ptr(), src.numel(), blocks, _stream_ptr(stream))
    if rc != GPT2_OK:
        raise GPT2Error(rc, "gpt2_probe_copy")
