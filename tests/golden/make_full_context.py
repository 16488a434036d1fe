"""Write the oracle's ten-step trajectory at a full-context workload, sampled.

    python tests/golden/make_full_context.py 124m|350m [--threads N] [--out PATH]

Test infrastructure: calls only the oracle and the seeded generators.  A float64 run
over ten AdamW steps of GPT-2 124M at B=8, T=1024 (or 350M at B=4, T=1024) is far too
long to repeat inside a test, so this script runs it once, in float64 and in float32,
and stores what the GPU test compares against:

  losses64 / losses32      mean loss at each of the ten steps (float64 / float32 oracle)
  <tensor>.pidx, .p        a sample of each parameter tensor after the ten updates
                           (float64 oracle values at 512 seeded uniform indices)
  <tensor>.ptop, .pt       the same at the 32 elements where the float32 oracle lands
                           furthest from the float64 one
  <tensor>.gidx, .g, .gtop, .gt   the same for the gradient of the tenth step
  pstats / gstats          per tensor, over the whole tensor: max |float64 value|, the
                           float32 oracle's max and 99th-percentile error relative to it

Each step's batch gradient is formed from single-row oracle runs (the mean loss over the
batch is the mean of the rows' mean losses; tests/parity.py, oracle_rowwise_gradient).
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
from scratch_transformer_lm_amd import synthetic as S  # noqa: E402
from tests.parity import oracle_rowwise_gradient  # noqa: E402

WORKLOADS = {"124m": S.GPT2_124M, "350m": S.GPT2_350M}
STEPS = 10
SAMPLE_UNIFORM = 512
SAMPLE_TOP = 32
SAMPLE_SEED = 5


def golden_path(key: str) -> str:
    return os.path.join(HERE, f"full_context_{key}.npz")


def trajectory(w, precision: str, steps: int):
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    m = O.OracleGPT2(w.model, 1, w.T, params, precision)
    losses = []
    grads = None
    for t in range(1, steps + 1):
        t0 = time.time()
        loss, _ = oracle_rowwise_gradient(m, x, y)
        losses.append(loss)
        if t == steps:
            grads = m.grads.astype(np.float64)
        assert m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t) == 0
        print(f"[{precision}] step {t} loss {loss:.9f} ({time.time() - t0:.0f} s)", flush=True)
    p = m.params.astype(np.float64)
    m.close()
    return np.array(losses), grads, p


def sample(rng, n: int, err: np.ndarray):
    uni = np.sort(rng.choice(n, size=min(SAMPLE_UNIFORM, n), replace=False)).astype(np.int64)
    top = np.sort(np.argsort(err, kind="stable")[-SAMPLE_TOP:]).astype(np.int64)
    return uni, top


def stats(ref: np.ndarray, other: np.ndarray):
    scale = float(np.max(np.abs(ref)))
    err = np.abs(other - ref) / max(scale, 1e-300)
    return scale, float(np.max(err)), float(np.percentile(err, 99)), err


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("workload", choices=sorted(WORKLOADS))
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--out", default=None, help="output path (default: next to this script)")
    a = ap.parse_args()
    w = WORKLOADS[a.workload]
    for prec in ("f64", "f32"):
        if a.threads:
            O.set_threads(a.threads, prec)
    l64, g64, p64 = trajectory(w, "f64", STEPS)
    l32, g32, p32 = trajectory(w, "f32", STEPS)
    offsets, lengths = O.param_layout(w.model)
    rng = np.random.default_rng(SAMPLE_SEED)
    out = {"workload": np.array(w.name), "steps": np.array(STEPS),
           "losses64": l64, "losses32": l32}
    pstats, gstats = [], []
    for name, o, n in zip(O.PARAM_NAMES, offsets, lengths):
        ps, pmax, p99, perr = stats(p64[o:o + n], p32[o:o + n])
        gs, gmax, g99, gerr = stats(g64[o:o + n], g32[o:o + n])
        (pidx, ptop), (gidx, gtop) = sample(rng, n, perr), sample(rng, n, gerr)
        out[f"{name}.pidx"], out[f"{name}.p"] = pidx, p64[o:o + n][pidx]
        out[f"{name}.ptop"], out[f"{name}.pt"] = ptop, p64[o:o + n][ptop]
        out[f"{name}.gidx"], out[f"{name}.g"] = gidx, g64[o:o + n][gidx]
        out[f"{name}.gtop"], out[f"{name}.gt"] = gtop, g64[o:o + n][gtop]
        pstats.append((ps, pmax, p99))
        gstats.append((gs, gmax, g99))
        print(f"{name}: params f32 err max {pmax:.2e} p99 {p99:.2e}; step-{STEPS} grads f32 err max "
              f"{gmax:.2e} p99 {g99:.2e}", flush=True)
    out["pstats"] = np.array(pstats)
    out["gstats"] = np.array(gstats)
    path = a.out or golden_path(a.workload)
    np.savez_compressed(path, **out)
    print("wrote", path, flush=True)


if __name__ == "__main__":
    main()
