"""GPU parity: the HIP library (through its C ABI) against the float64 CPU oracle.

Every test here runs kernels on the GPU and is marked `gpu`.  Inputs come from the
seeded generators; expected values come from the oracle only.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
from scipy.special import logsumexp

from scratch_transformer_lm_amd import synthetic as S
from tests.parity import (F32_FACTOR, GRAD_TOL, LN_BWD_TOL, LN_FWD_TOL, LOSS_RTOL, PARAM_TOL, oracle_rowwise_gradient,
                          param_bound, param_p99_bound, per_tensor, per_tensor_p99, rel_max, rel_p99, run_oracle)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from scratch_transformer_lm_amd import gpt2
    gpt2.load()
    return gpt2


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ LayerNorm alone

@pytest.mark.parametrize("N,C", [(8192, 768), (1, 64), (37, 1024), (5, 4), (130, 2048), (0, 768), (2049, 768)])
def test_layernorm_standalone(G, N, C):
    say(f"[layernorm] N={N} C={C}")
    from oracle import oracle as O
    if (N, C) == (8192, 768):
        x, w, b, dy = S.layernorm_inputs()
    else:
        x, w, b, dy = S.layernorm_inputs(N, C, seed=100 + N + C)
    tx, tw, tb, tdy = dev(x), dev(w), dev(b), dev(dy)
    y = torch.empty_like(tx)
    mean = torch.empty(N, device="cuda")
    rstd = torch.empty(N, device="cuda")
    G.layernorm_forward(y, mean, rstd, tx, tw, tb, 1e-5)
    dx = torch.full_like(tx, float("nan"))
    dw = torch.full_like(tw, float("nan"))
    db = torch.full_like(tb, float("nan"))
    ws = torch.full((max(1, G.layernorm_backward_workspace(N, C)),), float("nan"), device="cuda")
    G.layernorm_backward(dx, dw, db, tdy, tx, tw, mean, rstd, ws)
    if N == 0:
        assert np.all(host(dw) == 0) and np.all(host(db) == 0)
        return
    ry, rm, rr = O.layernorm_forward(x, w, b, 1e-5)
    rdx, rdw, rdb = O.layernorm_backward(dy, x, w, rm, rr)
    errs = dict(y=rel_max(host(y), ry), mean=rel_max(host(mean), rm), rstd=rel_max(host(rstd), rr),
                dx=rel_max(host(dx), rdx), dw=rel_max(host(dw), rdw), db=rel_max(host(db), rdb))
    say(errs)
    for k in ("y", "mean", "rstd"):
        assert errs[k] <= LN_FWD_TOL, k
    for k in ("dx", "dw", "db"):
        assert errs[k] <= LN_BWD_TOL, k


# ------------------------------------------------------------------ full training step

def gpu_run(G, w, params, x, y, steps, capture=(1,), B=None, T=None, variant=0):
    B = B or x.shape[0]
    T = T or x.shape[1]
    m = G.GPT2(w.model, B, T, variant=variant)
    m.params.copy_(dev(params))
    tx, ty = dev(x, torch.int32), dev(y, torch.int32)
    losses, grads = [], {}
    for t in range(1, steps + 1):
        losses.append(m.forward(tx, ty))
        assert m.last_error() == 0, G.strerror(m.last_error())
        assert m.zero_grad() == 0
        assert m.backward() == 0
        if t in capture:
            grads[t] = host(m.grads).copy()
        assert m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t) == 0
    return dict(losses=np.array(losses), grads=grads, params=host(m.params).copy(), model=m)


def check_training(G, w, steps, variant=0, B=None, T=None):
    """GPU against the float64 oracle: losses, every gradient tensor at steps 1 and last,
    every parameter tensor after the run.  In the mixed-precision variant the bfloat16
    rounding of each matmul operand is a step function of a value that fp32 and fp64
    compute slightly differently, so an element close to a rounding boundary may round
    one bf16 unit apart; there the loss and gradient bounds are, like the parameters',
    max(fixed tolerance, F32_FACTOR x the error of the oracle's own float32 build)."""
    params = S.init_params(w.model)
    x, y = S.tokens(w, B=B, T=T)
    bf = bool(variant & G.VARIANT_BF16)
    say(f"[train] {w.name} B={x.shape[0]} T={x.shape[1]} steps={steps} variant={variant}")
    gr = gpu_run(G, w, params, x, y, steps, capture=(1, steps), variant=variant)
    say("[train] gpu done; running oracle (float64, then float32)")
    orc = run_oracle(w, params, x, y, steps, capture_steps=(1, steps), variant=variant)
    o32 = run_oracle(w, params, x, y, steps, capture_steps=(1, steps) if bf else (), precision="f32",
                     variant=variant)
    m = gr["model"]
    loss_err = np.abs(gr["losses"] - orc["losses"]) / np.abs(orc["losses"])
    loss_tol = LOSS_RTOL
    if bf:
        loss_tol = max(LOSS_RTOL, F32_FACTOR * float(np.max(np.abs(o32["losses"] - orc["losses"]) / orc["losses"])))
    say("loss gpu", gr["losses"].tolist())
    say("loss ora", orc["losses"].tolist())
    say("loss rel err", loss_err.tolist(), "bound", loss_tol)
    bad = []
    for t in (1, steps):
        e = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, gr["grads"][t], orc["grads"][t])
        say(f"grad rel err step {t}:", {k: f"{v:.2e}" for k, v in e.items()})
        tol = {k: GRAD_TOL for k in e}
        if bf:
            e32g = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, o32["grads"][t], orc["grads"][t])
            say(f"float32 oracle grad rel err step {t}:", {k: f"{v:.2e}" for k, v in e32g.items()})
            tol = {k: max(GRAD_TOL, F32_FACTOR * e32g[k]) for k in e}
        bad += [(t, k, v, tol[k]) for k, v in e.items() if not v <= tol[k]]
        if bf:
            # the bulk of each gradient tensor: its 99th-percentile element error within
            # the fixed tolerance, or F32_FACTOR x the float32 oracle's own percentile
            # (after a few steps the bf16 rounding flips of earlier updates spread)
            q = per_tensor_p99(G.PARAM_NAMES, m.offsets, m.lengths, gr["grads"][t], orc["grads"][t])
            q32 = per_tensor_p99(G.PARAM_NAMES, m.offsets, m.lengths, o32["grads"][t], orc["grads"][t])
            say(f"grad p99 rel err step {t}:", {k: f"{v:.2e}" for k, v in q.items()})
            say(f"float32 oracle grad p99 rel err step {t}:", {k: f"{v:.2e}" for k, v in q32.items()})
            bad += [(t, "p99", k, v, q32[k]) for k, v in q.items() if not v <= max(GRAD_TOL, F32_FACTOR * q32[k])]
    e = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, gr["params"], orc["params"])
    e32 = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, o32["params"], orc["params"])
    say("param rel err:", {k: f"{v:.2e}" for k, v in e.items()})
    say("float32 oracle param rel err:", {k: f"{v:.2e}" for k, v in e32.items()})
    if not bf:
        q = per_tensor_p99(G.PARAM_NAMES, m.offsets, m.lengths, gr["params"], orc["params"])
        q32 = per_tensor_p99(G.PARAM_NAMES, m.offsets, m.lengths, o32["params"], orc["params"])
        say("param p99 rel err:", {k: f"{v:.2e}" for k, v in q.items()})
        say("float32 oracle param p99 rel err:", {k: f"{v:.2e}" for k, v in q32.items()})
        say("tensors above the literal 1e-4 (max, p99):",
            {k: (f"{e[k]:.1e}", f"{q[k]:.1e}") for k in e if e[k] > PARAM_TOL or q[k] > PARAM_TOL})
        bad += [("params", k, v, e32[k]) for k, v in e.items() if not v <= param_bound(e32[k])]
        bad += [("params p99", k, v, q32[k]) for k, v in q.items() if not v <= param_p99_bound(q32[k])]
    else:
        # AdamW moves every element by about lr per step whatever its gradient's size, so
        # an element whose gradient lies within bf16 rounding noise of zero (many bias
        # elements, whose parameters start at 0) may step either way in either run: the
        # largest single-element difference is noise.  Checked instead: the mean error of
        # each tensor against the float32 oracle's (a stable statistic over its elements),
        # and that no element is further apart than 3 lr per step.
        cap = 3.0 * w.lr * steps
        for k, o, n in zip(G.PARAM_NAMES, m.offsets, m.lengths):
            ref = orc["params"][o:o + n]
            scale = max(float(np.max(np.abs(ref))), 1e-30)
            mean_g = float(np.mean(np.abs(gr["params"][o:o + n] - ref))) / scale
            mean_32 = float(np.mean(np.abs(o32["params"][o:o + n] - ref))) / scale
            worst = float(np.max(np.abs(gr["params"][o:o + n] - ref)))
            if not (mean_g <= max(1e-5, F32_FACTOR * mean_32) and worst <= cap):
                bad.append(("params", k, mean_g, mean_32, worst, cap))
    assert np.all(loss_err <= loss_tol), loss_err
    assert not bad, bad


def test_tiny_forward_activations(G):
    w = S.TINY
    say(f"[activations] {w.name}")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T)
    m.params.copy_(dev(params))
    loss = m.forward(dev(x, torch.int32), dev(y, torch.int32))
    from oracle import oracle as O
    o = O.OracleGPT2(w.model, w.B, w.T, params)
    lo = o.forward(x, y)
    errs = {}
    for name in ("encoded", "lnf", "lnf_mean", "lnf_rstd", "losses"):
        errs[name] = rel_max(host(m.activation(name)).reshape(-1), o.activation(name))
    logits = o.activation("logits").reshape(w.B * w.T, -1)
    errs["logits"] = rel_max(host(m.activation("logits")), logits)
    errs["logits_lse"] = rel_max(host(m.activation("logits_lse")).reshape(-1), logsumexp(logits, axis=1))
    for l in range(w.model.num_layers):
        for name in ("ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "residual2", "ln2", "fch",
                     "fch_gelu", "residual3"):
            errs[f"{name}[{l}]"] = rel_max(host(m.activation(name, l)).reshape(-1), o.activation(name, l))
    say({k: f"{v:.1e}" for k, v in errs.items()})
    assert abs(loss - lo) / lo <= LOSS_RTOL
    assert max(errs.values()) <= 1e-5, errs


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_tiny_ten_steps(G, wd):
    import dataclasses
    check_training(G, dataclasses.replace(S.TINY, weight_decay=wd), 10)


def test_gpt2_124m_short_ten_steps(G):
    check_training(G, S.GPT2_124M_SHORT, 10)


@pytest.mark.parametrize("tiles", ["128", "96"])
@pytest.mark.parametrize("wl", ["tiny", "124m_short"])
def test_gemm_tile_widths(G, tiles, wl):
    """Every forward and dgrad matmul forced to one tile width (the automatic choice only
    takes 96-wide tiles at whole rounds of the grid): ragged column edges, split tiles and
    their fix-ups, and the dlogits dgrad at both widths, three steps against the oracle."""
    w = S.TINY if wl == "tiny" else S.GPT2_124M_SHORT
    G.set_gemm_tiles(G.GEMM_TILES_128 if tiles == "128" else G.GEMM_TILES_96)
    try:
        say(f"[gemm tiles {tiles}]")
        check_training(G, w, 3)
    finally:
        G.set_gemm_tiles(G.GEMM_TILES_AUTO)


# (workload, variant) pairs for the schedule tests: the base model, and the mixed-precision
# variant both at the same shape and where its weight gradients run as split-K rounds
SPLIT_K_SHAPE = S.Workload("gpt2 L1 C512 H8 V512 B4 T1024", S.ModelShape(1024, 512, 1, 8, 512), 4, 1024)
SCHEDULE_CASES = [("124m", 0), ("124m", 4), ("split-k", 4)]


def schedule_workload(name):
    return S.GPT2_124M_SHORT if name == "124m" else SPLIT_K_SHAPE


@pytest.mark.parametrize("wl,variant", SCHEDULE_CASES)
def test_backward_stream_schedules_agree_bitwise(G, wl, variant):
    """The default backward overlaps the weight gradients on a second stream; the
    single-stream schedule runs the same kernels in one order.  Two steps each: losses,
    gradients and updated parameters must be bitwise equal (in the mixed-precision
    variant this also covers the bf16 copies that the stream events order)."""
    w = schedule_workload(wl)
    say(f"[backward streams] {w.name} variant {variant}")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    runs = []
    for streams in (2, 1):
        m = G.GPT2(w.model, w.B, w.T, variant=variant)
        m.set_backward_streams(streams)
        m.params.copy_(dev(params))
        tx, ty = dev(x, torch.int32), dev(y, torch.int32)
        losses, grads = [], []
        for t in (1, 2):
            losses.append(m.forward(tx, ty))
            assert m.zero_grad() == 0 and m.backward() == 0, G.strerror(m.last_error())
            grads.append(host(m.grads).copy())
            assert m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t) == 0
        runs.append((losses, grads, host(m.params).copy()))
        m.close()
    (l2, g2, p2), (l1, g1, p1) = runs
    assert l2 == l1
    for a, b in zip(g2, g1):
        assert np.array_equal(a, b)
    assert np.array_equal(p2, p1)


# ------------------------------------------------------------------ sampling (sample_mult)

SAMPLE_SLACK = 2e-6  # coin distance from a cumulative boundary within which either side may differ


def sample_valid(probs, coin, token, slack=None):
    """`token` is the oracle's sample_mult pick, or a neighbour the coin is within
    SAMPLE_SLACK of (the GPU forms fp32 probabilities; the oracle's are float64)."""
    from oracle import oracle as O
    slack = SAMPLE_SLACK if slack is None else slack
    if token == O.sample_mult(probs, coin):
        return True
    cdf = np.cumsum(np.asarray(probs, dtype=np.float64))
    lo = cdf[token - 1] if token > 0 else 0.0
    return 0 <= token < len(probs) and lo - slack <= coin < cdf[token] + slack


def test_sample_matches_oracle(G):
    """gpt2_sample over a no-target forward at the 124M shape (V = 50257, B=4, T=64):
    rows spread over the batch, seeded coins plus the edges 0 and just below 1."""
    from oracle import oracle as O
    w = S.GPT2_124M_SHORT
    say("[sample]")
    params = S.init_params(w.model)
    x, _ = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T)
    m.params.copy_(dev(params))
    assert m.forward(dev(x, torch.int32), None) == -1.0
    rng = np.random.default_rng(21)
    rows = np.concatenate([[0, w.B * w.T - 1, 63, 64], rng.integers(0, w.B * w.T, 28)]).astype(np.int32)
    coins = np.concatenate([[0.0, 0.9999999, 0.5, 0.25], rng.random(28)]).astype(np.float32)
    toks = m.sample(rows, coins)
    o = O.OracleGPT2(w.model, w.B, w.T, params)
    assert o.forward(x, None) < 0
    probs = o.activation("probs").reshape(w.B * w.T, -1)
    exact = 0
    for r, c, t in zip(rows, coins, toks):
        assert sample_valid(probs[r], float(c), int(t)), (r, c, t, O.sample_mult(probs[r], float(c)))
        exact += int(t) == O.sample_mult(probs[r], float(c))
    say(f"sampled {len(rows)} rows, {exact} identical to the oracle's picks")
    assert exact >= len(rows) - 1
    # error paths: coin 1.0, row outside the forward, more requests than rows
    with pytest.raises(G.GPT2Error):
        m.sample([0], [1.0])
    with pytest.raises(G.GPT2Error):
        m.sample([w.B * w.T], [0.5])
    with pytest.raises(G.GPT2Error):
        m.sample(np.zeros(w.B * w.T + 1, np.int32), np.zeros(w.B * w.T + 1, np.float32))


def test_sample_needs_a_forward(G):
    w = S.TINY
    m = G.GPT2(w.model, w.B, w.T)
    with pytest.raises(G.GPT2Error) as e:
        m.sample([0], [0.5])
    assert e.value.code == G.GPT2_ESTATE


@pytest.mark.parametrize("variant", [0, 4])
def test_generate_matches_oracle(G, variant):
    """gpt2_generate on the tiny model from the end-of-text token (V-1): every generated
    token is checked against the oracle run on the GPU's own prefix, so one boundary
    coin cannot derail the rest of the comparison.  The forwards run on 1..39 rows, below
    every tile size.  In the mixed-precision variant a bf16 rounding flip can move a
    logit by up to 2^-7 of one product term (the tiny model's logits are O(0.1)), so a
    coin within 1e-3 of the oracle's cumulative probability counts as a boundary."""
    from oracle import oracle as O
    w = S.TINY
    say(f"[generate] variant {variant}")
    params = S.init_params(w.model)
    V = w.model.vocab_size
    total = 40
    coins = np.random.default_rng(33).random(total).astype(np.float32)
    m = G.GPT2(w.model, w.B, w.T, variant=variant)
    m.params.copy_(dev(params))
    toks = m.generate([V - 1], total, coins)
    assert toks[0] == V - 1 and np.all((toks >= 0) & (toks < V))
    o = O.OracleGPT2(w.model, 1, total - 1, params, variant=variant)
    slack = SAMPLE_SLACK if variant == 0 else 1e-3
    exact = 0
    for t in range(1, total):
        o.forward(toks[None, :t], None)
        p = o.activation("probs").reshape(1 * t, -1)[t - 1]
        assert sample_valid(p, float(coins[t - 1]), int(toks[t]), slack), t
        exact += int(toks[t]) == O.sample_mult(p, float(coins[t - 1]))
    say(f"generated {total - 1} tokens, {exact} identical to the oracle's picks")
    assert exact >= total - 2
    with pytest.raises(G.GPT2Error):
        m.generate([V - 1], w.model.max_seq_len + 1, np.zeros(w.model.max_seq_len + 1))


# ------------------------------------------------------------------ Llama-style variants

@pytest.mark.parametrize("variant", [1, 2, 3])
def test_variant_tiny_ten_steps(G, variant):
    """RMSNorm (1), rotary positions (2) and both (3): ten steps of the tiny model with
    weight decay against the oracle's variant, every gradient tensor at steps 1 and 10."""
    import dataclasses
    check_training(G, dataclasses.replace(S.TINY, weight_decay=0.1), 10, variant=variant)


def test_variant_124m_short_three_steps(G):
    check_training(G, S.GPT2_124M_SHORT, 3, variant=3)


def test_variant_tiny_forward_activations(G):
    """Both variants: RMSNorm outputs, their zero mean slots, the rotated qkv and every
    later activation against the oracle."""
    from oracle import oracle as O
    w = S.TINY
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T, variant=3)
    m.params.copy_(dev(params))
    loss = m.forward(dev(x, torch.int32), dev(y, torch.int32))
    o = O.OracleGPT2(w.model, w.B, w.T, params, variant=3)
    lo = o.forward(x, y)
    errs = {}
    for name in ("encoded", "lnf", "lnf_rstd", "losses"):
        errs[name] = rel_max(host(m.activation(name)).reshape(-1), o.activation(name))
    for l in range(w.model.num_layers):
        errs[f"qkv[{l}]"] = rel_max(host(m.activation("qkv", l)).reshape(-1), o.activation("qkv_rot", l))
        for name in ("ln1", "ln1_rstd", "atty", "residual2", "ln2", "fch_gelu", "residual3"):
            errs[f"{name}[{l}]"] = rel_max(host(m.activation(name, l)).reshape(-1), o.activation(name, l))
        assert not np.any(host(m.activation("ln1_mean", l)))
    say({k: f"{v:.1e}" for k, v in errs.items()})
    assert abs(loss - lo) / lo <= LOSS_RTOL
    assert max(errs.values()) <= 1e-5, errs


@pytest.mark.parametrize("wl,variant", SCHEDULE_CASES)
def test_backward_update_is_backward_then_update_bitwise(G, wl, variant):
    """gpt2_backward_update (each layer's AdamW as soon as its gradients are final) against
    gpt2_backward + gpt2_update, with both backward schedules: losses, gradients, params
    and both moments bitwise equal after three steps with weight decay."""
    w = schedule_workload(wl)
    say(f"[backward_update] {w.name} variant {variant}")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    runs = []
    for fused, streams in ((False, 2), (True, 2), (True, 1)):
        m = G.GPT2(w.model, w.B, w.T, variant=variant)
        m.set_backward_streams(streams)
        m.params.copy_(dev(params))
        tx, ty = dev(x, torch.int32), dev(y, torch.int32)
        losses = []
        for t in (1, 2, 3):
            losses.append(m.forward(tx, ty))
            assert m.zero_grad() == 0
            if fused:
                assert m.backward_update(w.lr, w.beta1, w.beta2, w.eps, 0.1, t) == 0
            else:
                assert m.backward() == 0
                assert m.update(w.lr, w.beta1, w.beta2, w.eps, 0.1, t) == 0
        runs.append((losses, host(m.grads).copy(), host(m.params).copy(), host(m.m).copy(), host(m.v).copy()))
        m.close()
    ref = runs[0]
    for r in runs[1:]:
        assert r[0] == ref[0]
        for a, b in zip(r[1:], ref[1:]):
            assert np.array_equal(a, b)


def test_gpt2_124m_ragged_shape(G):
    """The 124M model at B=3, T=100 (300 rows): ragged row edges in every GEMM at the real
    widths (128x96 and 128x128 tiles, split tiles and fix-ups) and a ragged last attention
    tile, one step against the oracle, every gradient and parameter tensor."""
    check_training(G, S.GPT2_124M_SHORT, 1, B=3, T=100)


@pytest.mark.parametrize("heads", [4, 2])
@pytest.mark.parametrize("variant", [0, 4])
def test_head_sizes_multi_tile(G, heads, variant):
    """Head sizes 16 and 32 (C=64 with 4 or 2 heads) at T=80: two query/key tiles, the
    second ragged, in the fp32 and the mixed-precision attention kernels; three steps
    against the oracle."""
    w = S.Workload(f"gpt2 L2 C64 H{heads} V512 B2 T80", S.ModelShape(128, 512, 2, heads, 64), 2, 80)
    check_training(G, w, 3, variant=variant)


def test_smaller_batch_than_built(G):
    w = S.TINY
    say("[smaller batch]")
    params = S.init_params(w.model)
    x, y = S.tokens(w, B=3, T=17, seed=7)
    gr = gpu_run(G, w, params, x, y, 2, capture=(2,), B=4, T=32)
    orc = run_oracle(w, params, x, y, 2, capture_steps=(2,))
    assert np.all(np.abs(gr["losses"] - orc["losses"]) / orc["losses"] <= LOSS_RTOL)
    m = gr["model"]
    e = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, gr["grads"][2], orc["grads"][2])
    assert max(e.values()) <= GRAD_TOL, e


@pytest.mark.parametrize("heads,C,Tb", [(4, 64, 64), (2, 128, 64)])
def test_attention_backward_recompute_path(G, heads, C, Tb):
    """A handle built at one sequence of Tb = 64 tokens sizes its score-gradient buffer for
    that sequence's one tile pair per head; called with two sequences of 32 tokens (the same
    token count, two tile pairs per head) the backward takes the path whose dQ kernel
    recomputes S and dP.  Head sizes 16 and 64, two steps against the oracle."""
    w = S.Workload(f"gpt2 L2 C{C} H{heads} V512", S.ModelShape(128, 512, 2, heads, C), 2, Tb // 2)
    say(f"[recompute path] C{C} H{heads}: built B1 T{Tb}, run B2 T{Tb // 2}")
    params = S.init_params(w.model)
    x, y = S.tokens(w, B=2, T=Tb // 2, seed=11)
    gr = gpu_run(G, w, params, x, y, 2, capture=(1, 2), B=1, T=Tb)
    orc = run_oracle(w, params, x, y, 2, capture_steps=(1, 2))
    assert np.all(np.abs(gr["losses"] - orc["losses"]) / orc["losses"] <= LOSS_RTOL)
    m = gr["model"]
    for t in (1, 2):
        e = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, gr["grads"][t], orc["grads"][t])
        say(f"grad rel err step {t}:", {k: f"{v:.1e}" for k, v in e.items()})
        assert max(e.values()) <= GRAD_TOL, e
    # the kernels that ran: the recomputing dQ, not the stored-score-gradient one
    m.profile_enable(True)
    m.forward(dev(x, torch.int32), dev(y, torch.int32))
    assert m.zero_grad() == 0 and m.backward() == 0
    torch.cuda.synchronize()
    names = {e["name"] for e in m.profile_entries()}
    m.profile_enable(False)
    hs = C // heads
    assert f"attn_bwd_dq_kernel<{hs}>" in names and f"attn_bwd_dq_ds_kernel<{hs}>" not in names, sorted(names)


@pytest.mark.parametrize("B,T", [(520, 64), (512, 64)])
def test_embedding_backward_paths(G, B, T):
    """B*T = 33280 takes the embedding backward's first-occurrence fallback (more positions
    than its one-block sort holds), B*T = 32768 the largest sorted batch; one step against
    the oracle, every gradient tensor."""
    w = S.TINY
    say(f"[embedding backward] B={B} T={T}")
    params = S.init_params(w.model)
    x, y = S.tokens(w, B=B, T=T, seed=11)
    gr = gpu_run(G, w, params, x, y, 1, capture=(1,))
    orc = run_oracle(w, params, x, y, 1, capture_steps=(1,))
    assert np.all(np.abs(gr["losses"] - orc["losses"]) / orc["losses"] <= LOSS_RTOL)
    m = gr["model"]
    e = per_tensor(G.PARAM_NAMES, m.offsets, m.lengths, gr["grads"][1], orc["grads"][1])
    say({k: f"{v:.1e}" for k, v in e.items()})
    assert max(e.values()) <= GRAD_TOL, e


# ------------------------------------------------------------------ full context (sampled)

def full_context_check(G, w, rows, variant=0):
    """One step at the full shape: sampled per-position losses against the oracle run on
    single rows, then properties that hold at any size: the gradient is the derivative of
    the GPU's own loss along the gradient, both embeddings receive the same total
    gradient, and the first AdamW step has a closed form.

    Mixed-precision variant: each sampled row's bound is max(LOSS_RTOL, F32_FACTOR x the
    error of the oracle's own float32 build on that row) (bf16 rounding flips, as in
    check_training); conservation holds exactly only when every row of the logits'
    gradient sums to zero, which its bf16 rounding breaks slightly (measured 5e-5, the
    same 1e-3 bound applies); and the directional derivative may differ by 1e-2 (the
    straight-through backward differs from the exact derivative by about the 3e-3
    gradient error the oracle itself shows)."""
    from oracle import oracle as O
    bf = bool(variant & G.VARIANT_BF16)
    say(f"[full] {w.name} variant {variant}")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T, variant=variant)
    m.params.copy_(dev(params))
    tx, ty = dev(x, torch.int32), dev(y, torch.int32)
    loss = m.forward(tx, ty)
    assert m.last_error() == 0
    losses = host(m.activation("losses")).reshape(w.B, w.T)
    assert abs(loss - losses.astype(np.float64).mean()) <= 1e-6 * loss
    for r in rows:
        say(f"[full] oracle row {r}")
        o = O.OracleGPT2(w.model, 1, w.T, params, forward_only=True, variant=variant)
        o.forward(x[r:r + 1], y[r:r + 1])
        ref = o.activation("losses")
        err = rel_max(losses[r], ref)
        tol = LOSS_RTOL
        o.close()
        del o
        if bf:
            o32 = O.OracleGPT2(w.model, 1, w.T, params, "f32", forward_only=True, variant=variant)
            o32.forward(x[r:r + 1], y[r:r + 1])
            tol = max(LOSS_RTOL, F32_FACTOR * rel_max(o32.activation("losses"), ref))
            o32.close()
            del o32
        say(f"row {r}: per-position loss rel err {err:.2e} (bound {tol:.2e})")
        assert err <= tol
    m.zero_grad()
    assert m.backward() == 0
    g = m.grads.clone()
    # conservation: sum over wte rows of dwte == sum over positions of dwpe
    off, ln = m.offsets, m.lengths
    C = w.model.channels
    s_wte = g[off[0]: off[0] + ln[0]].view(-1, C).double().sum(0)
    s_wpe = g[off[1]: off[1] + ln[1]].view(-1, C).double().sum(0)
    cons = float((s_wte - s_wpe).abs().max() / s_wpe.abs().max())
    say(f"embedding conservation rel err {cons:.2e}")
    assert cons <= 1e-3
    # directional derivative along the gradient, with the GPU's own fp32 forward; the
    # step moves the loss by about 0.02, far above fp32 noise (~1e-5) and small enough
    # that the curvature term stays below 1e-4 of the slope
    gn = float(g.double().norm())
    h = 1e-2 / (gn * gn)
    p0 = m.params.clone()
    m.params.copy_(p0 + h * g)
    lp = m.forward(tx, ty)
    m.params.copy_(p0 - h * g)
    lm = m.forward(tx, ty)
    m.params.copy_(p0)
    fd = (lp - lm) / (2 * h)
    say(f"fd {fd:.6e} vs |g|^2 {gn * gn:.6e}")
    assert abs(fd - gn * gn) <= (1e-2 if bf else 5e-3) * gn * gn
    # first AdamW step: p1 = p0 - lr (g/(|g|+eps) + wd p0)
    assert m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1) == 0
    gd, pd = g.double(), p0.double()
    ref = pd - w.lr * (gd / (gd.abs() + w.eps) + w.weight_decay * pd)
    err = float((m.params.double() - ref).abs().max() / pd.abs().max())
    say(f"adamw step-1 closed form rel err {err:.2e}")
    assert err <= 1e-6


# ------------------------------------------------------------------ full context vs the oracle
#
# GPT-2 124M at B=8, T=1024 (the benchmarked shape) and 350M at B=4, T=1024 (weight decay
# 0.1), compared element by element with the float64 oracle.  The oracle's batch gradient
# is formed from single-row runs (tests/parity.py, oracle_rowwise_gradient).  Step 1 is
# compared live: every position's loss and every element of every gradient tensor.  The
# ten-step trajectory takes the float64 oracle far too long to repeat here, so it comes
# from tests/golden/full_context_<key>.npz, written by tests/golden/make_full_context.py
# (oracle only): the loss of every step, and samples of the tenth step's gradients and of
# the parameters after ten updates, with the float32 oracle's whole-tensor errors.

FULL_CONTEXT = {"124m": S.GPT2_124M, "350m": S.GPT2_350M}
FULL_STEPS = 10
_full_gpu = {}


def full_context_gpu(G, key):
    """Ten GPU steps of a full-context workload (kept for the two tests of that workload):
    losses, step-1 per-position losses, gradients of steps 1 and 10, final parameters."""
    if key in _full_gpu:
        return _full_gpu[key]
    _full_gpu.clear()
    w = FULL_CONTEXT[key]
    say(f"[full context] {w.name}: {FULL_STEPS} GPU steps")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T)
    m.params.copy_(dev(params))
    tx, ty = dev(x, torch.int32), dev(y, torch.int32)
    out = dict(losses=[], offsets=m.offsets, lengths=m.lengths)
    for t in range(1, FULL_STEPS + 1):
        out["losses"].append(m.forward(tx, ty))
        assert m.last_error() == 0, G.strerror(m.last_error())
        if t == 1:
            out["per_pos"] = host(m.activation("losses")).reshape(w.B, w.T).copy()
        assert m.zero_grad() == 0 and m.backward() == 0
        if t in (1, FULL_STEPS):
            out[f"g{t}"] = host(m.grads).copy()
        assert m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t) == 0
    out["losses"] = np.array(out["losses"])
    out["params"] = host(m.params).copy()
    m.close()
    _full_gpu[key] = out
    return out


def full_context_step1(G, key):
    """Step 1 against the live float64 oracle: the mean loss, every row's per-position
    losses (1e-5 relative to the row's largest), every gradient tensor element-wise."""
    from oracle import oracle as O
    w = FULL_CONTEXT[key]
    gpu = full_context_gpu(G, key)
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    say(f"[full context] {w.name}: float64 oracle, {w.B} single-row runs")
    o = O.OracleGPT2(w.model, 1, w.T, params)
    loss, per_pos = oracle_rowwise_gradient(o, x, y, progress=lambda r: say(f"  oracle row {r} done"))
    lerr = abs(gpu["losses"][0] - loss) / loss
    say(f"loss gpu {gpu['losses'][0]:.9f} oracle {loss:.9f} rel err {lerr:.2e}")
    row_err = [rel_max(gpu["per_pos"][r], per_pos[r]) for r in range(w.B)]
    say("per-position loss rel err by row:", [f"{e:.1e}" for e in row_err])
    e = per_tensor(G.PARAM_NAMES, gpu["offsets"], gpu["lengths"], gpu["g1"], o.grads)
    q = per_tensor_p99(G.PARAM_NAMES, gpu["offsets"], gpu["lengths"], gpu["g1"], o.grads)
    say("grad rel err step 1:", {k: f"{v:.2e}" for k, v in e.items()})
    say("grad p99 rel err step 1:", {k: f"{v:.2e}" for k, v in q.items()})
    o.close()
    assert lerr <= LOSS_RTOL
    assert max(row_err) <= LOSS_RTOL, row_err
    assert max(e.values()) <= GRAD_TOL, e


def full_context_ten_steps(G, key):
    """Ten steps against the stored float64 trajectory: every step's loss (1e-5); the
    tenth step's gradients on the stored sample (largest error 1e-3); the parameters on
    the stored sample (largest error within param_bound of the float32 oracle's largest
    whole-tensor error, the uniform sample's 99th percentile within param_p99_bound of the
    float32 oracle's whole-tensor percentile)."""
    import os
    w = FULL_CONTEXT[key]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"full_context_{key}.npz")
    assert os.path.exists(path), f"{path} missing: run python tests/golden/make_full_context.py {key}"
    gold = np.load(path, allow_pickle=False)
    assert str(gold["workload"]) == w.name and int(gold["steps"]) == FULL_STEPS
    gpu = full_context_gpu(G, key)
    _full_gpu.clear()
    lerr = np.abs(gpu["losses"] - gold["losses64"]) / gold["losses64"]
    l32 = np.abs(gold["losses32"] - gold["losses64"]) / gold["losses64"]
    say("loss gpu", gpu["losses"].tolist())
    say("loss oracle", gold["losses64"].tolist())
    say("loss rel err", [f"{v:.1e}" for v in lerr], "float32 oracle", [f"{v:.1e}" for v in l32])
    bad = []
    rows = []
    for i, (k, o, n) in enumerate(zip(G.PARAM_NAMES, gpu["offsets"], gpu["lengths"])):
        ps, p32max, p32p99 = gold["pstats"][i]
        gs, g32max, g32p99 = gold["gstats"][i]
        pu, gu = gpu["params"][o:o + n], gpu["g10"][o:o + n]
        eu = np.abs(pu[gold[f"{k}.pidx"]] - gold[f"{k}.p"]) / ps
        et = np.abs(pu[gold[f"{k}.ptop"]] - gold[f"{k}.pt"]) / ps
        pmax, pp99 = float(max(eu.max(), et.max())), float(np.percentile(eu, 99))
        gu_e = np.abs(gu[gold[f"{k}.gidx"]] - gold[f"{k}.g"]) / gs
        gt_e = np.abs(gu[gold[f"{k}.gtop"]] - gold[f"{k}.gt"]) / gs
        gmax = float(max(gu_e.max(), gt_e.max()))
        rows.append(f"{k}: params max {pmax:.1e} (f32 {p32max:.1e}) p99 {pp99:.1e} (f32 {p32p99:.1e}); "
                    f"grads max {gmax:.1e} (f32 {g32max:.1e})")
        if not pmax <= param_bound(p32max):
            bad.append(("params max", k, pmax, p32max))
        if not pp99 <= param_p99_bound(p32p99):
            bad.append(("params p99", k, pp99, p32p99))
        if not gmax <= GRAD_TOL:
            bad.append(("grads step 10", k, gmax, g32max))
    for r in rows:
        say(r)
    assert np.all(lerr <= LOSS_RTOL), lerr
    assert not bad, bad


@pytest.mark.timeout(400)
def test_gpt2_124m_full_context_step1(G):
    full_context_step1(G, "124m")


@pytest.mark.timeout(400)
def test_gpt2_124m_full_context_ten_steps(G):
    full_context_ten_steps(G, "124m")


@pytest.mark.timeout(400)
def test_gpt2_350m_full_context_step1(G):
    full_context_step1(G, "350m")


@pytest.mark.timeout(400)
def test_gpt2_350m_full_context_ten_steps(G):
    full_context_ten_steps(G, "350m")


def test_bf16_124m_full_context(G):
    """The mixed-precision variant at the shape and launch configuration the benchmark
    times (124M, B=8, T=1024)."""
    full_context_check(G, S.GPT2_124M, rows=(0, 7), variant=G.VARIANT_BF16)


# ------------------------------------------------------------------ ABI behaviour on GPU

def test_errors_accumulation_and_determinism(G):
    w = S.TINY
    say("[abi]")
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T)
    m.params.copy_(dev(params))
    tx, ty = dev(x, torch.int32), dev(y, torch.int32)
    assert m.backward() == G.GPT2_ESTATE
    assert m.update(1e-4, 0.9, 0.999, 1e-8, 0.0, 0) == G.GPT2_ESTATE
    bad = tx.clone()
    bad[1, 5] = 512
    assert math.isnan(m.forward(bad, ty)) and m.last_error() == G.GPT2_EINVAL
    badt = ty.clone()
    badt[0, 0] = -3
    assert math.isnan(m.forward(tx, badt)) and m.last_error() == G.GPT2_EINVAL
    assert m.backward() == G.GPT2_ESTATE
    assert math.isnan(m.forward(dev(np.zeros((1, 65), np.int32)), None))
    assert m.forward(tx, None) == -1.0
    assert m.backward() == G.GPT2_ESTATE
    l1 = m.forward(tx, ty)
    m.zero_grad()
    m.backward()
    g1 = host(m.grads).copy()
    m.backward()
    g2 = host(m.grads).copy()
    assert rel_max(g2, 2 * g1) <= 1e-6
    m.zero_grad()
    l2 = m.forward(tx, ty)
    m.backward()
    assert l1 == l2 and np.array_equal(host(m.grads), g1)


def test_bf16_batch_shape_beyond_built_tiles(G):
    """The mixed-precision variant sizes its per-head attention copies in whole 64-position
    tiles of the built shape: built at (B=1, T=64), a forward at (B=2, T=32) has the same
    B*T but needs two tiles, and is refused before any launch; (1, 40) fits."""
    w = S.TINY
    say("[bf16 shape bound]")
    params = S.init_params(w.model)
    m = G.GPT2(w.model, 1, 64, variant=G.VARIANT_BF16)
    m.params.copy_(dev(params))
    x, y = S.tokens(w, B=2, T=32)
    assert math.isnan(m.forward(dev(x, torch.int32), dev(y, torch.int32)))
    assert m.last_error() == G.GPT2_EINVAL
    x1, y1 = S.tokens(w, B=1, T=40)
    loss = m.forward(dev(x1, torch.int32), dev(y1, torch.int32))
    assert m.last_error() == 0 and math.isfinite(loss)


# ------------------------------------------------------------------ mixed precision

@pytest.mark.parametrize("wl,steps,variant", [("tiny", 10, 4), ("tiny", 10, 7), ("124m", 3, 4)])
def test_bf16_training(G, wl, steps, variant):
    """Mixed-precision variant (bf16 matmul operands), alone and with RMSNorm + RoPE."""
    check_training(G, S.TINY if wl == "tiny" else S.GPT2_124M_SHORT, steps, variant=variant)


@pytest.mark.parametrize("variant", [4, 7])
def test_bf16_forward_activations(G, variant):
    """Every forward activation of the tiny bf16 model (attention on bf16 q, k, v with
    unrounded probabilities, then the bf16 linear layers) against the float64 oracle.
    A value that fp32 and fp64 compute slightly differently may round to bf16 one unit
    apart when it lies next to a rounding boundary; such a flip moves a product term by
    at most 2^-7 of itself.  So, per tensor: the 99th percentile of the element errors
    (relative to the tensor's largest value) within max(1e-5, F32_FACTOR x the oracle's
    float32 build's), and every element within 1e-2, far below what a wrong index,
    operand or scale gives."""
    from oracle import oracle as O
    w = S.TINY
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = G.GPT2(w.model, w.B, w.T, variant=variant)
    m.params.copy_(dev(params))
    loss = m.forward(dev(x, torch.int32), dev(y, torch.int32))
    o64 = O.OracleGPT2(w.model, w.B, w.T, params, variant=variant)
    o32 = O.OracleGPT2(w.model, w.B, w.T, params, "f32", variant=variant)
    l64, l32 = o64.forward(x, y), o32.forward(x, y)
    assert abs(loss - l64) / l64 <= max(LOSS_RTOL, F32_FACTOR * abs(l32 - l64) / l64)
    def p99(a, ref):
        ref = np.asarray(ref, np.float64).reshape(-1)
        d = np.abs(np.asarray(a, np.float64).reshape(-1) - ref) / max(np.max(np.abs(ref)), 1e-30)
        return float(np.percentile(d, 99)), float(np.max(d))

    bad = []
    for l in range(w.model.num_layers):
        for name in ("ln1", "qkv", "atty", "residual2", "ln2", "fch_gelu", "residual3"):
            oname = "qkv_rot" if name == "qkv" and variant & G.VARIANT_ROPE else name  # GPU keeps it rotated
            ref = o64.activation(oname, l)
            e99, emax = p99(host(m.activation(name, l)), ref)
            f99, fmax = p99(o32.activation(oname, l), ref)
            say(f"{name}[{l}] p99 {e99:.1e} max {emax:.1e} (float32 oracle p99 {f99:.1e} max {fmax:.1e})")
            if not (e99 <= max(1e-5, F32_FACTOR * f99) and emax <= 1e-2):
                bad.append((name, l, e99, emax, f99))
    assert not bad, bad


def test_bf16_split_k_weight_gradients(G):
    """One layer at C=512 with B*T = 4096: the fc and fcproj weight gradients (64 output
    tiles, k = 4096) run as 8-way split-K rounds, k-segment first, with the segment
    partials added by the split-K fix-up (the full-size shapes take this path too)."""
    check_training(G, SPLIT_K_SHAPE, 1, variant=G.VARIANT_BF16)


def test_bf16_ragged_shape(G):
    """bf16 variant at the 124M widths with 300 rows: the weight gradients' last k-tile
    (300 = 4 x 64 + 44 rows, filled with zeros past row 300) and ragged GEMM edges."""
    check_training(G, S.GPT2_124M_SHORT, 1, variant=G.VARIANT_BF16, B=3, T=100)
