"""gpt2_layernorm_backward_noalloc (the allocation-free LayerNorm backward) against
gpt2_layernorm_backward with a caller workspace, through the C ABI, on the GPU.

Two calls in a row on one device, the second on a smaller input: both must give the
workspace call's results bitwise (the same kernels run) and meet the oracle's LayerNorm
tolerances, so partial rows the first call left in the fixed scratch cannot leak into
the second."""
from __future__ import annotations

import numpy as np
import pytest

from scratch_transformer_lm_amd import synthetic as S
from tests.parity import LN_BWD_TOL, rel_max

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _case(G, N, C, seed):
    from oracle import oracle as O
    x, w, b, dy = S.layernorm_inputs(N, C, seed=seed)
    tx, tw, tb, tdy = (torch.from_numpy(a).cuda() for a in (x, w, b, dy))
    y = torch.empty_like(tx)
    mean = torch.empty(N, device="cuda")
    rstd = torch.empty(N, device="cuda")
    G.layernorm_forward(y, mean, rstd, tx, tw, tb, 1e-5)
    outs = []
    for noalloc in (False, True):
        dx = torch.full_like(tx, float("nan"))
        dw = torch.full_like(tw, float("nan"))
        db = torch.full_like(tb, float("nan"))
        if noalloc:
            G.layernorm_backward_noalloc(dx, dw, db, tdy, tx, tw, mean, rstd)
        else:
            ws = torch.full((max(1, G.layernorm_backward_workspace(N, C)),), float("nan"), device="cuda")
            G.layernorm_backward(dx, dw, db, tdy, tx, tw, mean, rstd, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (dx, dw, db)])
    ref_fwd = O.layernorm_forward(x, w, b, 1e-5)
    ref = O.layernorm_backward(dy, x, w, ref_fwd[1], ref_fwd[2])
    return outs, ref


def test_noalloc_layernorm_backward_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from scratch_transformer_lm_amd import gpt2 as G
    G.load()
    assert G.layernorm_backward_noalloc_max_floats() >= G.layernorm_backward_workspace(8192, 768)
    for N, C, seed in ((8192, 768, 2), (300, 256, 7)):  # second call smaller
        print(f"[noalloc] N={N} C={C}", flush=True)
        (ws, na), ref = _case(G, N, C, seed)
        for a, b in zip(ws, na):
            assert np.array_equal(a, b)
        errs = [rel_max(a, r) for a, r in zip(na, ref)]
        print(f"dx dw db rel err vs oracle: {errs}", flush=True)
        assert max(errs) <= LN_BWD_TOL
    # a request beyond the fixed scratch is refused before any launch (C > 4096 is
    # refused as an argument error first)
    t = torch.zeros(4, 8192, device="cuda")
    v = torch.zeros(8192, device="cuda")
    s = torch.zeros(4, device="cuda")
    with pytest.raises(G.GPT2Error) as e:
        G.layernorm_backward_noalloc(t, v, v, t, t, v, s, s)
    assert e.value.code == G.GPT2_EINVAL
