"""ctypes wrapper of the CPU oracle (gpt2_oracle.c).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module; the GPU library and its binding never do.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

from . import build as _build

PARAM_NAMES = ("wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb")
ACT_NAMES = ("encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "preatt", "att", "attproj",
             "residual2", "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "fcproj", "residual3",
             "lnf", "lnf_mean", "lnf_rstd", "logits", "probs", "losses")
PER_LAYER = set(ACT_NAMES[1:17])
# Model variants (bit mask): RMSNorm for every LayerNorm, rotary q/k positions (the
# Llama-style layers), and mixed precision (bfloat16-rounded matmul operands).
VARIANT_RMSNORM, VARIANT_ROPE, VARIANT_BF16 = 1, 2, 4


class Config(ct.Structure):
    _fields_ = [("max_seq_len", ct.c_int), ("vocab_size", ct.c_int), ("num_layers", ct.c_int),
                ("num_heads", ct.c_int), ("channels", ct.c_int)]


_LIBS: dict[str, ct.CDLL] = {}


def load(precision: str = "f64") -> ct.CDLL:
    if precision in _LIBS:
        return _LIBS[precision]
    path = _build.lib_path(precision)
    if not os.path.exists(path):
        if precision.endswith("_native"):
            _build.build_native(precision[:-len("_native")])
        else:
            _build.build()
    lib = ct.CDLL(path)
    real = ct.c_double if precision.startswith("f64") else ct.c_float
    P = ct.c_void_p
    sz = ct.c_size_t
    i = ct.c_int
    lib.oracle_real_size.restype = i
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_get_threads.restype = i
    lib.oracle_gpt2_num_parameters.argtypes = [ct.POINTER(Config)]
    lib.oracle_gpt2_num_parameters.restype = sz
    lib.oracle_gpt2_param_layout.argtypes = [ct.POINTER(Config), P, P]
    lib.oracle_gpt2_param_layout.restype = i
    lib.oracle_gpt2_num_activations.argtypes = [ct.POINTER(Config), i, i]
    lib.oracle_gpt2_num_activations.restype = sz
    lib.oracle_gpt2_build.argtypes = [ct.POINTER(P), ct.POINTER(Config), i, i, P, P, P, P]
    lib.oracle_gpt2_build_variant.argtypes = [ct.POINTER(P), ct.POINTER(Config), i, i, P, P, P, P, i]
    lib.oracle_gpt2_build.restype = i
    lib.oracle_gpt2_free.argtypes = [P]
    lib.oracle_gpt2_last_error.argtypes = [P]
    lib.oracle_gpt2_last_error.restype = i
    lib.oracle_gpt2_forward.argtypes = [P, P, P, i, i]
    lib.oracle_gpt2_forward.restype = ct.c_double
    lib.oracle_gpt2_zero_grad.argtypes = [P]
    lib.oracle_gpt2_zero_grad.restype = i
    lib.oracle_gpt2_backward.argtypes = [P]
    lib.oracle_gpt2_backward.restype = i
    lib.oracle_gpt2_update.argtypes = [P, real, real, real, real, real, i]
    lib.oracle_gpt2_update.restype = i
    lib.oracle_gpt2_activation.argtypes = [P, i, i, i, ct.POINTER(sz)]
    lib.oracle_gpt2_activation.restype = P
    lib.oracle_layernorm_forward.argtypes = [P, P, P, P, P, P, i, i, real]
    lib.oracle_layernorm_backward.argtypes = [P, P, P, P, P, P, P, P, i, i]
    lib.oracle_encoder_forward.argtypes = [P, P, P, P, i, i, i]
    lib.oracle_encoder_backward.argtypes = [P, P, P, P, i, i, i]
    lib.oracle_matmul_forward.argtypes = [P, P, P, P, i, i, i]
    lib.oracle_matmul_backward.argtypes = [P, P, P, P, P, P, i, i, i]
    lib.oracle_attention_forward.argtypes = [P, P, P, P, i, i, i, i]
    lib.oracle_attention_backward.argtypes = [P, P, P, P, P, P, i, i, i, i]
    lib.oracle_gelu_forward.argtypes = [P, P, sz]
    lib.oracle_gelu_backward.argtypes = [P, P, P, sz]
    lib.oracle_residual_forward.argtypes = [P, P, P, sz]
    lib.oracle_residual_backward.argtypes = [P, P, P, sz]
    lib.oracle_softmax_forward.argtypes = [P, P, i, i]
    lib.oracle_sample_mult.argtypes = [P, i, real]
    lib.oracle_rmsnorm_forward.argtypes = [P, P, P, P, i, i, real]
    lib.oracle_rmsnorm_backward.argtypes = [P, P, P, P, P, P, i, i]
    lib.oracle_rope_forward.argtypes = [P, P, i, i, i, i]
    lib.oracle_rope_backward.argtypes = [P, P, i, i, i, i]
    lib.oracle_sample_mult.restype = i
    lib.oracle_crossentropy_forward.argtypes = [P, P, P, i, i]
    lib.oracle_crossentropy_softmax_backward.argtypes = [P, P, P, P, i, i]
    lib.oracle_adamw.argtypes = [P, P, P, P, sz, real, real, real, real, real, i]
    lib.oracle_bf16_round.argtypes = [real]
    lib.oracle_bf16_round.restype = real
    lib.oracle_bf16_round_array.argtypes = [P, P, sz]
    _LIBS[precision] = lib
    return lib


def dtype_of(precision: str):
    """f64, f32 (portable builds) or f32_native / f64_native (built for the host)."""
    return np.float64 if precision.startswith("f64") else np.float32


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


def config(shape) -> Config:
    """Config from any object with the five GPT-2 config fields."""
    return Config(shape.max_seq_len, shape.vocab_size, shape.num_layers, shape.num_heads,
                  shape.channels)


def num_parameters(shape, precision: str = "f64") -> int:
    c = config(shape)
    return load(precision).oracle_gpt2_num_parameters(ct.byref(c))


def num_activations(shape, B: int, T: int, precision: str = "f64") -> int:
    c = config(shape)
    return load(precision).oracle_gpt2_num_activations(ct.byref(c), B, T)


def param_layout(shape, precision: str = "f64"):
    c = config(shape)
    off = np.zeros(16, np.uint64)
    ln = np.zeros(16, np.uint64)
    rc = load(precision).oracle_gpt2_param_layout(ct.byref(c), _ptr(off), _ptr(ln))
    if rc != 0:
        raise ValueError(f"oracle_gpt2_param_layout: {rc}")
    return [int(x) for x in off], [int(x) for x in ln]


def set_threads(n: int, precision: str = "f64") -> None:
    load(precision).oracle_set_threads(n)


class OracleGPT2:
    """The oracle model: owns numpy params/grads/m/v in the oracle's precision."""

    def __init__(self, shape, B: int, T: int, params: np.ndarray, precision: str = "f64",
                 forward_only: bool = False, variant: int = 0):
        self.lib = load(precision)
        self.precision = precision
        self.dtype = dtype_of(precision)
        self.shape = shape
        self.cfg = config(shape)
        n = self.lib.oracle_gpt2_num_parameters(ct.byref(self.cfg))
        if params.size != n:
            raise ValueError(f"params has {params.size} elements, model needs {n}")
        self.params = np.ascontiguousarray(params, dtype=self.dtype).copy()
        if forward_only:
            self.grads = self.m = self.v = None
        else:
            self.grads = np.zeros(n, self.dtype)
            self.m = np.zeros(n, self.dtype)
            self.v = np.zeros(n, self.dtype)
        h = ct.c_void_p()
        rc = self.lib.oracle_gpt2_build_variant(ct.byref(h), ct.byref(self.cfg), B, T, _ptr(self.params),
                                                _ptr(self.grads), _ptr(self.m), _ptr(self.v), variant)
        if rc != 0:
            raise ValueError(f"oracle_gpt2_build failed: {rc}")
        self.h = h
        self.offsets, self.lengths = param_layout(shape, precision)
        self._keep = []

    def close(self):
        if self.h:
            self.lib.oracle_gpt2_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def last_error(self) -> int:
        return self.lib.oracle_gpt2_last_error(self.h)

    def forward(self, inputs: np.ndarray, targets: np.ndarray | None) -> float:
        inputs = np.ascontiguousarray(inputs, dtype=np.int32)
        B, T = inputs.shape
        tg = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32)
        self._keep = [inputs, tg]
        return self.lib.oracle_gpt2_forward(self.h, _ptr(inputs), _ptr(tg), B, T)

    def zero_grad(self) -> int:
        return self.lib.oracle_gpt2_zero_grad(self.h)

    def backward(self) -> int:
        return self.lib.oracle_gpt2_backward(self.h)

    def update(self, lr, beta1, beta2, eps, weight_decay, t) -> int:
        return self.lib.oracle_gpt2_update(self.h, lr, beta1, beta2, eps, weight_decay, t)

    def tensor(self, buf: np.ndarray, name: str) -> np.ndarray:
        i = PARAM_NAMES.index(name)
        return buf[self.offsets[i]: self.offsets[i] + self.lengths[i]]

    def activation(self, name: str, layer: int = 0, grad: bool = False) -> np.ndarray:
        cnt = ct.c_size_t()
        aid = len(ACT_NAMES) if name == "qkv_rot" else ACT_NAMES.index(name)  # rotary variant only
        p = self.lib.oracle_gpt2_activation(self.h, aid, layer, int(grad), ct.byref(cnt))
        if not p:
            raise ValueError(f"no activation {name}[{layer}]")
        buf = (ct.c_double if self.precision.startswith("f64") else ct.c_float) * cnt.value
        return np.frombuffer(buf.from_address(p), dtype=self.dtype).copy()


# ---- layer hooks on numpy arrays (allocate outputs, call the C layer) --------------

def _real(a, precision):
    return np.ascontiguousarray(a, dtype=dtype_of(precision))


def layernorm_forward(x, w, b, eps=1e-5, precision="f64"):
    lib = load(precision)
    x, w, b = (_real(a, precision) for a in (x, w, b))
    N, C = x.shape
    y = np.empty_like(x)
    mean = np.empty(N, x.dtype)
    rstd = np.empty(N, x.dtype)
    lib.oracle_layernorm_forward(_ptr(y), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(w), _ptr(b), N, C, eps)
    return y, mean, rstd


def layernorm_backward(dy, x, w, mean, rstd, precision="f64"):
    """Overwrite semantics: returns fresh (dx, dw, db)."""
    lib = load(precision)
    dy, x, w, mean, rstd = (_real(a, precision) for a in (dy, x, w, mean, rstd))
    N, C = x.shape
    dx = np.zeros_like(x)
    dw = np.zeros(C, x.dtype)
    db = np.zeros(C, x.dtype)
    lib.oracle_layernorm_backward(_ptr(dx), _ptr(dw), _ptr(db), _ptr(dy), _ptr(x), _ptr(w),
                                  _ptr(mean), _ptr(rstd), N, C)
    return dx, dw, db


def attention_forward(qkv, NH, precision="f64"):
    lib = load(precision)
    qkv = _real(qkv, precision)
    B, T, C3 = qkv.shape
    C = C3 // 3
    out = np.empty((B, T, C), qkv.dtype)
    pre = np.empty((B, NH, T, T), qkv.dtype)
    att = np.empty((B, NH, T, T), qkv.dtype)
    lib.oracle_attention_forward(_ptr(out), _ptr(pre), _ptr(att), _ptr(qkv), B, T, C, NH)
    return out, pre, att


def attention_backward(dout, qkv, att, NH, precision="f64"):
    lib = load(precision)
    dout, qkv, att = (_real(a, precision) for a in (dout, qkv, att))
    B, T, C3 = qkv.shape
    C = C3 // 3
    dqkv = np.zeros_like(qkv)
    dpre = np.zeros_like(att)
    datt = np.zeros_like(att)
    lib.oracle_attention_backward(_ptr(dqkv), _ptr(dpre), _ptr(datt), _ptr(dout), _ptr(qkv),
                                  _ptr(att), B, T, C, NH)
    return dqkv, dpre, datt


def gelu_forward(x, precision="f64"):
    lib = load(precision)
    x = _real(x, precision)
    y = np.empty_like(x)
    lib.oracle_gelu_forward(_ptr(y), _ptr(x), x.size)
    return y


def gelu_backward(x, dy, precision="f64"):
    lib = load(precision)
    x, dy = _real(x, precision), _real(dy, precision)
    dx = np.zeros_like(x)
    lib.oracle_gelu_backward(_ptr(dx), _ptr(x), _ptr(dy), x.size)
    return dx


def matmul_forward(x, w, bias=None, precision="f64"):
    lib = load(precision)
    x, w = _real(x, precision), _real(w, precision)
    bias = None if bias is None else _real(bias, precision)
    N, IC = x.shape
    OC = w.shape[0]
    out = np.empty((N, OC), x.dtype)
    lib.oracle_matmul_forward(_ptr(out), _ptr(x), _ptr(w), _ptr(bias), N, IC, OC)
    return out


def matmul_backward(dout, x, w, with_bias=True, precision="f64"):
    lib = load(precision)
    dout, x, w = (_real(a, precision) for a in (dout, x, w))
    N, IC = x.shape
    OC = w.shape[0]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    db = np.zeros(OC, x.dtype) if with_bias else None
    lib.oracle_matmul_backward(_ptr(dx), _ptr(dw), _ptr(db), _ptr(dout), _ptr(x), _ptr(w), N, IC, OC)
    return dx, dw, db


def bf16_round(x, precision="f64"):
    """Each element rounded to the nearest bfloat16 value (ties to even)."""
    lib = load(precision)
    x = _real(np.asarray(x), precision)
    out = np.empty_like(x)
    lib.oracle_bf16_round_array(_ptr(out), _ptr(x), x.size)
    return out


def softmax_forward(logits, precision="f64"):
    lib = load(precision)
    z = _real(logits, precision)
    N, V = z.shape
    p = np.empty_like(z)
    lib.oracle_softmax_forward(_ptr(p), _ptr(z), N, V)
    return p


def rmsnorm_forward(x, w, eps=1e-5, precision="f64"):
    lib = load(precision)
    x = _real(x, precision)
    N, C = x.shape
    y = np.empty_like(x)
    r = np.empty(N, dtype=x.dtype)
    lib.oracle_rmsnorm_forward(_ptr(y), _ptr(r), _ptr(x), _ptr(_real(w, precision)), N, C, eps)
    return y, r


def rmsnorm_backward(dy, x, w, rstd, precision="f64"):
    lib = load(precision)
    x = _real(x, precision)
    N, C = x.shape
    dx = np.zeros_like(x)
    dw = np.zeros(C, dtype=x.dtype)
    lib.oracle_rmsnorm_backward(_ptr(dx), _ptr(dw), _ptr(_real(dy, precision)), _ptr(x), _ptr(_real(w, precision)),
                                _ptr(_real(rstd, precision)), N, C)
    return dx, dw


def rope_forward(qkv, NH, precision="f64"):
    """qkv (B, T, 3C) -> the same with q and k rotated (v copied)."""
    lib = load(precision)
    x = _real(qkv, precision)
    B, T, C3 = x.shape
    y = np.empty_like(x)
    lib.oracle_rope_forward(_ptr(y), _ptr(x), B, T, C3 // 3, NH)
    return y


def rope_backward(dout, NH, precision="f64"):
    lib = load(precision)
    d = _real(dout, precision)
    B, T, C3 = d.shape
    dx = np.zeros_like(d)
    lib.oracle_rope_backward(_ptr(dx), _ptr(d), B, T, C3 // 3, NH)
    return dx


def sample_mult(probs, coin, precision="f64"):
    """Index drawn from the distribution `probs` (1-D) by the coin in [0, 1)."""
    lib = load(precision)
    p = _real(probs, precision).reshape(-1)
    return int(lib.oracle_sample_mult(_ptr(p), len(p), float(coin)))


def crossentropy_forward(probs, targets, precision="f64"):
    lib = load(precision)
    p = _real(probs, precision)
    tg = np.ascontiguousarray(targets, dtype=np.int32)
    N, V = p.shape
    out = np.empty(N, p.dtype)
    lib.oracle_crossentropy_forward(_ptr(out), _ptr(p), _ptr(tg), N, V)
    return out


def crossentropy_softmax_backward(dlosses, probs, targets, precision="f64"):
    lib = load(precision)
    p = _real(probs, precision)
    dl = _real(dlosses, precision)
    tg = np.ascontiguousarray(targets, dtype=np.int32)
    N, V = p.shape
    d = np.zeros_like(p)
    lib.oracle_crossentropy_softmax_backward(_ptr(d), _ptr(dl), _ptr(p), _ptr(tg), N, V)
    return d


def encoder_forward(tokens, wte, wpe, precision="f64"):
    lib = load(precision)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    wte, wpe = _real(wte, precision), _real(wpe, precision)
    B, T = tok.shape
    C = wte.shape[1]
    out = np.empty((B, T, C), wte.dtype)
    lib.oracle_encoder_forward(_ptr(out), _ptr(tok), _ptr(wte), _ptr(wpe), B, T, C)
    return out


def encoder_backward(dout, tokens, V, maxT, precision="f64"):
    lib = load(precision)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    dout = _real(dout, precision)
    B, T, C = dout.shape
    dwte = np.zeros((V, C), dout.dtype)
    dwpe = np.zeros((maxT, C), dout.dtype)
    lib.oracle_encoder_backward(_ptr(dwte), _ptr(dwpe), _ptr(dout), _ptr(tok), B, T, C)
    return dwte, dwpe


def adamw(p, g, m, v, lr, b1, b2, eps, wd, t, precision="f64"):
    """Returns updated (p, m, v) copies."""
    lib = load(precision)
    p, g, m, v = (_real(a, precision).copy() for a in (p, g, m, v))
    lib.oracle_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.size, lr, b1, b2, eps, wd, t)
    return p, m, v
