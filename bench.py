"""Training-step throughput of the GPT-2 fp32 step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload gpt2-124M B8 T1024]
                    [--no-cpu-baseline]

One step = gpt2_forward + gpt2_zero_grad + gpt2_backward + gpt2_update (AdamW) over one
synthetic batch already resident in HBM (the pages' forward / zero_grad / backward /
update loop on a single batch).  Prints ONE JSON line.  Besides throughput it reports
the roofline position of the kernel that takes the most time (measured with HIP events
around each of its launches, on the library's stream, over the timed region) and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from scratch_transformer_lm_amd import synthetic as S  # noqa: E402

PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12


def step_flops(m: S.ModelShape, B: int, T: int) -> float:
    """Algorithmic FLOPs of one training step: 2 per multiply-add, backward twice the
    forward, attention over the causal half only."""
    C, L, V = m.channels, m.num_layers, m.vocab_size
    BT = B * T
    linear = 2 * BT * (12 * C * C) * L + 2 * BT * C * V
    attn = L * B * 2 * 2 * (T * (T + 1) / 2) * C  # QK^T and PV over u <= t
    return 3.0 * (linear + attn)


def cpu_baseline(w: S.Workload, rows: int = 1):
    """The oracle (float64, as it stands) on a bounded sample: `rows` sequences of the
    workload, one full step (forward, zero_grad, backward, AdamW)."""
    from oracle import oracle as O
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    x, y = x[:rows], y[:rows]
    m = O.OracleGPT2(w.model, rows, w.T, params)
    t0 = time.perf_counter()
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1)
    dt = time.perf_counter() - t0
    threads = O.load().oracle_get_threads()
    m.close()
    return dict(value=rows * w.T / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{rows} sequence(s) of {w.T} tokens of the same workload, one full step "
                       f"(forward, zero_grad, backward, AdamW) in float64, {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=S.GPT2_124M.name)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); multi-GPU data "
              "parallelism is not part of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    from scratch_transformer_lm_amd import gpt2 as G
    w = S.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    model = G.GPT2(w.model, w.B, w.T, stream=stream)
    model.params.copy_(torch.from_numpy(S.init_params(w.model)).cuda())
    x, y = S.tokens(w)
    tx = torch.from_numpy(x).cuda()
    ty = torch.from_numpy(y).cuda()
    torch.cuda.synchronize()

    t = 0

    def step():
        nonlocal t
        t += 1
        loss = model.forward(tx, ty)
        model.zero_grad()
        model.backward()
        model.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
        return loss

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    prof = model.profile_enable(True) if hasattr(model, "profile_enable") else False
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    losses = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if model.last_error() != 0 or not all(np.isfinite(losses)):
        print(f"bench: step failed: {G.strerror(model.last_error())}, losses {losses}", file=sys.stderr)
        sys.exit(1)
    ms = dt * 1e3 / args.steps
    tokens = w.B * w.T
    flops = step_flops(w.model, w.B, w.T)
    out = {
        "metric": "training tokens/sec (fwd+bwd+AdamW), GPT-2 124M fp32, B=8 T=1024, 1 MI355X"
        if w is S.GPT2_124M else f"training tokens/sec (fwd+bwd+AdamW), {w.name} fp32, 1 MI355X",
        "value": tokens / (dt / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (Zipf(1.1) int32 tokens with separator 50256 every 256; N(0,0.02) init)",
        "config": {"workload": w.name, "global_batch": w.B, "seq_len": w.T,
                   "layers": w.model.num_layers, "channels": w.model.channels,
                   "heads": w.model.num_heads, "vocab": w.model.vocab_size,
                   "parallelism": "single GPU"},
        "tflops": flops / (dt / args.steps) / 1e12,
        "step_roofline_frac": flops / PEAK_FP32_MFMA / (dt / args.steps),
        "loss_first_last": [losses[0], losses[-1]],
    }
    if prof:
        out["roofline"], out["kernels"] = model.profile_report(args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
