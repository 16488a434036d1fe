"""Shared pieces of the GPU-vs-oracle parity tests.

Tolerances (GPU fp32 against the float64 oracle, per tensor, as "max abs difference
over max abs oracle value"):
  loss                           relative 1e-5 at every step
  every gradient tensor          1e-3 (steps 1 and last)
  parameters after the run       1e-4, or 4x the error of the oracle's own float32 build
                                 when that is larger (see param_bound)
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
