"""Seeded synthetic workloads: token streams, initial parameters, LayerNorm tensors.

This module is shared by the GPU path's harness and by the CPU oracle's tests, and
it holds none of the training step's arithmetic: it only draws numbers and lays them
out in the shapes the model expects.

Workload recipe (the pages train GPT-2 on GPT-2-tokenized text with pretrained
weights; neither is available, so these draws stand in for them):

* tokens: int32 ids (the pages' token files are raw int32 GPT-2 ids, llm.c README
  translation, "快速上手"), drawn i.i.d. from a Zipf(s=1.1) law over [0, V):
  p_k proportional to (k+1)^-1.1, token 0 the most frequent.  One stream of B*T+1
  ids is drawn; inputs are its first B*T ids, targets the same stream shifted by one.
  At V = 50257 the id 50256 (GPT-2's end-of-text id) overwrites every 256th position
  of the stream as a document separator; it masks nothing.
* parameters: the 16 GPT-2 tensors in their canonical order, row-major, weights
  (out, in).  wte, wpe, qkvw, fcw ~ N(0, 0.02); attprojw, fcprojw ~ N(0, 0.02/sqrt(2L));
  every bias 0; LayerNorm gamma 1, beta 0.  Drawn as float32 from one generator in
  tensor order.
* LayerNorm standalone tensors: x ~ N(0,1) (rows, C), gamma ~ N(1, 0.1),
  beta ~ N(0, 0.1), dy ~ N(0,1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TOKEN_SEED = 0
PARAM_SEED = 1
LAYERNORM_SEED = 2
SEPARATOR_ID = 50256
SEPARATOR_PERIOD = 256
ZIPF_S = 1.1

PARAM_NAMES = (
    "wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
    "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb",
)


@dataclasses.dataclass(frozen=True)
class ModelShape:
    max_seq_len: int
    vocab_size: int
    num_layers: int
    num_heads: int
    channels: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    B: int
    T: int
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    steps: int = 10
    separator: bool = False


def param_shapes(m: ModelShape):
    """Shapes of the 16 parameter tensors, in storage order."""
    V, C, L, T = m.vocab_size, m.channels, m.num_layers, m.max_seq_len
    return (
        (V, C), (T, C), (L, C), (L, C), (L, 3 * C, C), (L, 3 * C), (L, C, C), (L, C),
        (L, C), (L, C), (L, 4 * C, C), (L, 4 * C), (L, C, 4 * C), (L, C), (C,), (C,),
    )


def param_sizes(m: ModelShape):
    return tuple(int(np.prod(s)) for s in param_shapes(m))


# The workloads: a tiny model, the 124M model at the pages' own run shape
# (B*T = 256), the 124M model at full context, and the 350M model.
TINY = Workload("gpt2-tiny L2 C64 H4 V512 B2 T32", ModelShape(64, 512, 2, 4, 64), 2, 32)
GPT2_124M_SHORT = Workload("gpt2-124M B4 T64", ModelShape(1024, 50257, 12, 12, 768), 4, 64,
                           separator=True)
GPT2_124M = Workload("gpt2-124M B8 T1024", ModelShape(1024, 50257, 12, 12, 768), 8, 1024,
                     separator=True, steps=20)
GPT2_350M = Workload("gpt2-350M B4 T1024", ModelShape(1024, 50257, 24, 16, 1024), 4, 1024,
                     separator=True, weight_decay=0.1)
# Standalone LayerNorm: 8192 rows of 768 channels, eps 1e-5.
LAYERNORM_ROWS, LAYERNORM_C, LAYERNORM_EPS = 8192, 768, 1e-5

WORKLOADS = {w.name: w for w in (TINY, GPT2_124M_SHORT, GPT2_124M, GPT2_350M)}


def zipf_probs(V: int, s: float = ZIPF_S) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def token_stream(V: int, n: int, separator: bool, seed: int = TOKEN_SEED) -> np.ndarray:
    rng = np.random.default_rng(seed)
    s = rng.choice(V, size=n, p=zipf_probs(V)).astype(np.int32)
    if separator:
        s[::SEPARATOR_PERIOD] = SEPARATOR_ID
    return s


def tokens(w: Workload, B: int | None = None, T: int | None = None, seed: int = TOKEN_SEED):
    """(inputs, targets), each int32 (B, T), C-contiguous."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    s = token_stream(w.model.vocab_size, B * T + 1, w.separator, seed)
    inputs = np.ascontiguousarray(s[: B * T].reshape(B, T))
    targets = np.ascontiguousarray(s[1: B * T + 1].reshape(B, T))
    return inputs, targets


def init_params(m: ModelShape, seed: int = PARAM_SEED) -> np.ndarray:
    """One flat float32 buffer holding the 16 tensors in storage order."""
    rng = np.random.default_rng(seed)
    sizes = param_sizes(m)
    out = np.empty(sum(sizes), dtype=np.float32)
    resid_std = 0.02 / math.sqrt(2 * m.num_layers)
    off = 0
    for name, n in zip(PARAM_NAMES, sizes):
        view = out[off: off + n]
        if name in ("wte", "wpe", "qkvw", "fcw"):
            view[:] = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
        elif name in ("attprojw", "fcprojw"):
            view[:] = rng.standard_normal(n, dtype=np.float32) * np.float32(resid_std)
        elif name in ("ln1w", "ln2w", "lnfw"):
            view[:] = 1.0
        else:
            view[:] = 0.0
        off += n
    return out


def split_params(m: ModelShape, flat: np.ndarray):
    """Views of the flat buffer as the 16 named tensors."""
    out = {}
    off = 0
    for name, shape in zip(PARAM_NAMES, param_shapes(m)):
        n = int(np.prod(shape))
        out[name] = flat[off: off + n].reshape(shape)
        off += n
    return out


def layernorm_inputs(rows: int = LAYERNORM_ROWS, C: int = LAYERNORM_C, seed: int = LAYERNORM_SEED):
    """(x, gamma, beta, dy) as float32."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, C), dtype=np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32)
    dy = rng.standard_normal((rows, C), dtype=np.float32)
    return x, gamma, beta, dy
