"""Host-side checks of the HIP library (CPU only: no kernel runs).

The library must load, export every function include/gpt2.h declares, and its host
logic (parameter count and layout, arena sizes, argument checks) must agree with the
closed form and with the oracle.
"""
from __future__ import annotations

import ctypes as ct
import os

import pytest

from oracle import oracle as O
from scratch_transformer_lm_amd import gpt2 as G
from scratch_transformer_lm_amd import synthetic as S

pytestmark = pytest.mark.skipif(not os.path.exists(G.LIB_PATH), reason="library not built")


def test_every_declared_symbol_is_exported():
    lib = G.load()
    names = G.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n


def test_library_defines_every_internal_symbol():
    """A shared library links with unresolved symbols and fails only when loaded: every
    gpt2k:: function the library calls must be defined in it (weak TLS helpers aside)."""
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-C", "-u", G.LIB_PATH], capture_output=True, text=True, check=True).stdout
    missing = [l.strip() for l in out.splitlines()
               if ("gpt2k::" in l or "gpt2_" in l) and not l.split()[0] in ("w", "v")]
    assert not missing, missing


def closed_form(m):
    V, C, L, T = m.vocab_size, m.channels, m.num_layers, m.max_seq_len
    return V * C + T * C + L * (12 * C * C + 13 * C) + 2 * C


@pytest.mark.parametrize("w", [S.TINY, S.GPT2_124M, S.GPT2_350M])
def test_parameter_count_and_layout(w):
    assert G.num_parameters(w.model) == closed_form(w.model) == O.num_parameters(w.model)
    assert G.param_layout(w.model) == O.param_layout(w.model)


def test_printed_parameter_count():
    assert G.num_parameters(S.GPT2_124M.model) == 124439808


def test_bad_configs_rejected():
    bad = [S.ModelShape(64, 512, 2, 3, 64),    # C not a multiple of NH
           S.ModelShape(64, 512, 2, 1, 128),   # head size 128 unsupported
           S.ModelShape(64, 512, 0, 4, 64),    # no layers
           S.ModelShape(64, 512, 2, 2, 66)]    # C not a multiple of 4 (and head size 33)
    for m in bad:
        assert G.num_parameters(m) == 0
        with pytest.raises(G.GPT2Error):
            G.arena_sizes(m, 2, 32)


def test_arena_sizes():
    a, s = G.arena_sizes(S.TINY.model, 2, 32)
    assert a > 0 and s > 0
    a2, s2 = G.arena_sizes(S.TINY.model, 4, 32)
    assert a2 > a and s2 >= s
    with pytest.raises(G.GPT2Error):
        G.arena_sizes(S.TINY.model, 1, 65)          # T > max_seq_len
    a3, _ = G.arena_sizes(S.GPT2_124M.model, 8, 1024)
    # no (B,NH,T,T) score tensors: far below the plain inventory at full context
    assert a3 < O.num_activations(S.GPT2_124M.model, 8, 1024) / 2


def test_build_argument_checks_need_no_gpu():
    lib = G.load()
    cfg = G.config(S.TINY.model)
    h = ct.c_void_p()
    bufs = G.Buffers()
    assert lib.gpt2_build(ct.byref(h), ct.byref(cfg), 2, 32, ct.byref(bufs), None) == G.GPT2_EINVAL
    assert lib.gpt2_build(None, ct.byref(cfg), 2, 32, ct.byref(bufs), None) == G.GPT2_EINVAL
    assert lib.gpt2_forward(None, None, None, 1, 1) != lib.gpt2_forward(None, None, None, 1, 1)  # NaN
    assert lib.gpt2_backward(None) == G.GPT2_EINVAL
    assert lib.gpt2_layernorm_forward(None, None, None, None, None, None, 4, 8, 1e-5, None) == G.GPT2_EINVAL
    assert lib.gpt2_layernorm_backward_workspace(8192, 768) >= 2 * 768
    assert G.strerror(G.GPT2_ESTATE) == "call out of order"


def test_gemm_tile_policy_values():
    lib = G.load()
    for bad in (-1, 3, 96):
        assert lib.gpt2_set_gemm_tiles(bad) == G.GPT2_EINVAL
    for ok in (G.GEMM_TILES_128, G.GEMM_TILES_96, G.GEMM_TILES_AUTO):
        assert lib.gpt2_set_gemm_tiles(ok) == G.GPT2_OK
    with pytest.raises(G.GPT2Error):
        G.set_gemm_tiles(5)


def test_backward_streams_argument_checks():
    lib = G.load()
    assert lib.gpt2_set_backward_streams(None, 2) == G.GPT2_EINVAL
    assert lib.gpt2_set_backward_streams(None, 1) == G.GPT2_EINVAL


def test_sampling_argument_checks_need_no_gpu():
    lib = G.load()
    assert lib.gpt2_sample(None, None, None, 1, None) == G.GPT2_EINVAL
    assert lib.gpt2_generate(None, None, 1, 2, None) == G.GPT2_EINVAL


def test_build_variant_argument_checks_need_no_gpu():
    lib = G.load()
    cfg = G.config(S.TINY.model)
    h = ct.c_void_p()
    bufs = G.Buffers()
    assert lib.gpt2_build_variant(ct.byref(h), ct.byref(cfg), 2, 32, ct.byref(bufs), None, 8) == G.GPT2_EINVAL
    assert lib.gpt2_build_variant(ct.byref(h), ct.byref(cfg), 2, 32, ct.byref(bufs), None, 4) == G.GPT2_EINVAL
    assert lib.gpt2_build_variant(None, ct.byref(cfg), 2, 32, ct.byref(bufs), None, 3) == G.GPT2_EINVAL


@pytest.mark.parametrize("w,B,T", [(S.TINY, 2, 32), (S.GPT2_124M, 8, 1024), (S.GPT2_124M, 3, 100)])
def test_bf16_variant_arena_sizes(w, B, T):
    """The mixed-precision arenas hold at least the bf16 copies: weights straight and
    transposed, the four per-layer linear inputs and lnf; the scratch one copy per kind of
    output gradient (residual stream, fc, qkv) and the logits gradient's.  (The fp32
    scratch alone holds the attention backward's score gradients of one layer and the
    forward's raw scores of every layer: B heads' worth of 64x64 blocks for every causal
    pair of 64-row tiles each.)"""
    m = w.model
    L, C, V, NH = m.num_layers, m.channels, m.vocab_size, m.num_heads
    BT = B * T
    a0, s0 = G.arena_sizes(m, B, T)
    a4, s4 = G.arena_sizes(m, B, T, G.VARIANT_BF16)
    weights = L * 12 * C * C + V * C
    acts = L * 7 * C * BT + C * BT
    nqt = (T + 63) // 64
    ds = (L + 1) * B * NH * (nqt * (nqt + 1) // 2) * 4096
    assert s0 >= ds
    assert (a4 - a0) * 2 >= 2 * weights + acts
    assert (s4 - (s0 - ds)) * 2 >= 8 * C * BT + V * BT
    with pytest.raises(G.GPT2Error):
        G.arena_sizes(m, B, T, 8)


def test_backward_update_argument_checks_need_no_gpu():
    lib = G.load()
    assert lib.gpt2_backward_update(None, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1) == G.GPT2_EINVAL
