"""Shared pieces of the GPU-vs-oracle parity tests.

Tolerances (GPU fp32 against the float64 oracle, per tensor; an element's error is its
absolute difference over the tensor's largest absolute oracle value):
  loss                           relative 1e-5 at every step
  every gradient tensor          largest element error 1e-3 (steps 1 and last)
  parameters after the run       largest element error 1e-4, or 4x that of the oracle's own
                                 float32 build when larger (param_bound); and the 99th
                                 percentile of the element errors 1e-4, or 4x the float32
                                 build's 99th percentile when larger (param_p99_bound)
  LayerNorm standalone outputs   y, mean, rstd 1e-5;  dx, dgamma, dbeta 1e-3
"""
from __future__ import annotations

import numpy as np

LOSS_RTOL = 1e-5
GRAD_TOL = 1e-3
PARAM_TOL = 1e-4
LN_FWD_TOL = 1e-5
LN_BWD_TOL = 1e-3


F32_FACTOR = 4.0


def param_bound(f32_err: float) -> float:
    """Bound on a parameter tensor's error after a multi-step AdamW run.

    AdamW divides each gradient by its own magnitude plus eps, so elements whose
    gradient sits at rounding-noise level (exactly zero for the key bias, since softmax
    ignores a per-query constant, or below eps) move by an amount fp32 arithmetic cannot
    determine; on a repeated batch the trajectory also amplifies small differences.  The
    oracle's own float32 build, against its float64 build, shows how far float32
    arithmetic of the very same definition lands; the GPU must be within 1e-4 or within
    F32_FACTOR times that distance, whichever is larger."""
    return max(PARAM_TOL, F32_FACTOR * f32_err)


def param_p99_bound(f32_p99: float) -> float:
    """Bound on the 99th percentile of a parameter tensor's element errors after a
    multi-step AdamW run: 1e-4, or F32_FACTOR times the float32 oracle's own 99th
    percentile when larger.  Unlike the largest element error (set by the few elements
    whose gradient sits at the rounding-noise floor), the percentile is a stable
    statistic of the tensor: over six parameter seeds of the tiny model the float32
    build's own value varies by 1.2-4.1x per tensor."""
    return max(PARAM_TOL, F32_FACTOR * f32_p99)


def rel_p99(a, ref) -> float:
    """99th percentile of |a - ref| / max |ref| over the elements."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    if not ref.size:
        return 0.0
    den = float(np.max(np.abs(ref)))
    d = np.abs(a - ref)
    return float(np.percentile(d / den if den > 0 else d, 99))


def per_tensor_p99(names, offsets, lengths, a, ref):
    return {n: rel_p99(a[o:o + l], ref[o:o + l]) for n, o, l in zip(names, offsets, lengths)}


def rel_max(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(a - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def per_tensor(names, offsets, lengths, a, ref):
    return {n: rel_max(a[o:o + l], ref[o:o + l]) for n, o, l in zip(names, offsets, lengths)}


def run_oracle(w, params, inputs, targets, steps, capture_steps=(1,), precision="f64", variant=0):
    from oracle import oracle as O
    m = O.OracleGPT2(w.model, inputs.shape[0], inputs.shape[1], params, precision, variant=variant)
    losses, grads = [], {}
    for t in range(1, steps + 1):
        losses.append(m.forward(inputs, targets))
        m.zero_grad()
        assert m.backward() == 0
        if t in capture_steps:
            grads[t] = m.grads.copy()
        m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
    out = dict(losses=np.array(losses), grads=grads, params=m.params.copy(), model=m)
    return out


def oracle_rowwise_gradient(m, x, y, progress=None):
    """Full-batch losses and gradient of a (B, T) batch from single-row oracle runs.

    The mean loss over the B*T positions equals the mean over rows of each row's own
    mean loss, so its gradient is the mean of the rows' gradients.  The oracle's backward
    adds into its gradient buffer, so B single-row forward/backward pairs after one
    zero_grad leave the sum of the rows' gradients there, and scaling by 1/B gives the
    mean (a power-of-two scale, exact in floating point, for B = 4 and 8).  `m` is an
    oracle model built for one row of T positions.  Returns the mean loss (float64) and
    the (B, T) per-position losses."""
    B = x.shape[0]
    m.zero_grad()
    rows = []
    for r in range(B):
        m.forward(x[r:r + 1], y[r:r + 1])
        rows.append(m.activation("losses").astype(np.float64))
        assert m.backward() == 0
        if progress is not None:
            progress(r)
    m.grads *= m.dtype(1.0 / B)
    per_pos = np.stack(rows)
    return float(per_pos.mean()), per_pos
