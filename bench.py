"""Training-step throughput of the GPT-2 fp32 step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload gpt2-124M B8 T1024]
                    [--no-cpu-baseline]

One step = gpt2_forward + gpt2_zero_grad + gpt2_backward_update over one synthetic batch
already resident in HBM: the pages' forward / zero_grad / backward / update loop on a
single batch, with backward and the AdamW update in the library's fused call (bitwise
gpt2_backward followed by gpt2_update; it starts each layer's update as soon as that
layer's gradients are final).  Prints ONE JSON line.  Besides throughput it reports
the roofline position of the kernel that takes the most time (measured with HIP events
around each of its launches, on the stream that launch runs on, over the timed region;
plus the same kernel in a single-stream step) and the CPU oracle timed on a bounded
sample of the same workload.
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
PEAK_BF16_MFMA = 2.5e15  # dense
PEAK_HBM = 8.0e12


def mfma_peak(name: str) -> float:
    """Matrix-core peak of a kernel's arithmetic: bf16 for the mixed-precision GEMM."""
    return PEAK_BF16_MFMA if name.startswith("gemm_bf16_kernel") else PEAK_FP32_MFMA


def step_flops(m: S.ModelShape, B: int, T: int) -> float:
    """Algorithmic FLOPs of one training step: 2 per multiply-add, backward twice the
    forward, attention over the causal half only."""
    C, L, V = m.channels, m.num_layers, m.vocab_size
    BT = B * T
    linear = 2 * BT * (12 * C * C) * L + 2 * BT * C * V
    attn = L * B * 2 * 2 * (T * (T + 1) / 2) * C  # QK^T and PV over u <= t
    return 3.0 * (linear + attn)


def roofline(kernels):
    """Roofline position of the kernel with the largest total time: its algorithmic work
    per launch over its average launch duration, against the MI355X peak of its bound
    (the matrix cores of its data type for kernels that count flops, HBM otherwise)."""
    k = max(kernels, key=lambda e: e["ms"])
    avg_s = k["ms"] / k["launches"] / 1e3
    if k["flops"] > 0:
        achieved = k["flops"] / k["launches"] / avg_s / 1e12
        r = dict(bound="mfma", achieved=achieved, peak=mfma_peak(k["name"]) / 1e12, unit="TFLOP/s")
    else:
        achieved = k["bytes"] / k["launches"] / avg_s / 1e9
        r = dict(bound="hbm", achieved=achieved, peak=PEAK_HBM / 1e9, unit="GB/s")
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = None
    r["kernel"] = k["name"]
    r["launches"] = k["launches"]
    r["avg_launch_us"] = avg_s * 1e6
    return r


def breakdown(kernels, steps):
    out = []
    for k in sorted(kernels, key=lambda e: -e["ms"]):
        avg_s = k["ms"] / k["launches"] / 1e3
        e = dict(name=k["name"], ms_per_step=k["ms"] / steps, launches_per_step=k["launches"] / steps)
        if k["flops"] > 0:
            e["tflops"] = k["flops"] / k["launches"] / avg_s / 1e12
            e["frac_mfma"] = e["tflops"] * 1e12 / mfma_peak(k["name"])
        else:
            e["gbps"] = k["bytes"] / k["launches"] / avg_s / 1e9
            e["frac_hbm"] = e["gbps"] * 1e9 / PEAK_HBM
        out.append(e)
    return out


def kernel_source_digest(kernel: str) -> str:
    """Digest of the source file that defines `kernel` and of the shared kernel headers."""
    import hashlib
    csrc = os.path.join(ROOT, "scratch_transformer_lm_amd", "csrc")
    base = kernel.split("<")[0]
    files = sorted(f for f in os.listdir(csrc) if f.endswith(".hip")
                   and (base + "(") in open(os.path.join(csrc, f)).read())
    h = hashlib.sha256()
    for f in files + ["common.h", "kernels.h"]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    there is none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel") != kernel or rec.get("sources") != kernel_source_digest(kernel):
        return None
    return float(rec["traffic_bytes_per_launch"])


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
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain device copy of MIB MiB three times "
                         "(a kernel of known traffic for scaling hardware byte counters)")
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
        model.backward_update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
        return loss

    # Warm-up; all but the first warm-up step carry events around every kernel, which
    # gives the per-kernel breakdown and names the kernel that takes the most time.
    step()
    model.profile_enable(True)
    for _ in range(max(1, args.warmup - 1)):
        step()
    torch.cuda.synchronize()
    all_kernels = model.profile_entries()
    dominant = max(all_kernels, key=lambda e: e["ms"])["name"]
    # The timed region: K steps, with HIP events around each launch of the dominant kernel
    # only, recorded on the stream that launch runs on.
    model.profile_enable(True)
    model.profile_filter(dominant)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    losses = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kernels = model.profile_entries()
    model.profile_enable(False)
    # The same K steps without any events, to show what the events cost.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt_plain = time.perf_counter() - t1
    # One more step with the whole backward on one stream and events on every kernel: each
    # kernel's own rate, undisturbed by the overlapping weight-gradient stream.
    model.set_backward_streams(1)
    model.profile_enable(True)
    step()
    torch.cuda.synchronize()
    isolated = model.profile_entries()
    model.profile_enable(False)
    model.set_backward_streams(2)
    # Forward-only generation with the trained-for-K-steps weights (the pages' sample
    # loop): 64 new tokens from the end-of-text token, one fixed coin per token, each
    # step recomputing the whole prefix; the sampling kernel timed with events.
    gen_new = 64
    coins = np.random.default_rng(7).random(gen_new).astype(np.float32)
    eot = w.model.vocab_size - 1
    model.profile_enable(True)
    model.profile_filter("sample_kernel")
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    gen = model.generate([eot], gen_new + 1, coins)
    torch.cuda.synchronize()
    dt_gen = time.perf_counter() - t2
    sk = [e for e in model.profile_entries() if e["name"] == "sample_kernel"]
    model.profile_enable(False)
    # The Llama-style variant (RMSNorm + rotary positions) at the same shape: a second
    # model, 2 warm-up steps (the second with events on every kernel), 5 timed steps.
    vm = G.GPT2(w.model, w.B, w.T, stream=stream, variant=G.VARIANT_RMSNORM | G.VARIANT_ROPE)
    vm.params.copy_(model.params)
    tv = 0

    def vstep():
        nonlocal tv
        tv += 1
        loss = vm.forward(tx, ty)
        vm.zero_grad()
        vm.backward_update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, tv)
        return loss

    vstep()
    vm.profile_enable(True)
    vstep()
    torch.cuda.synchronize()
    vkernels = vm.profile_entries()
    vm.profile_enable(False)
    t3 = time.perf_counter()
    vlosses = [vstep() for _ in range(5)]
    torch.cuda.synchronize()
    dt_var = (time.perf_counter() - t3) / 5
    verr = vm.last_error()
    vm.close()
    if verr != 0 or not all(np.isfinite(vlosses)):
        print(f"bench: variant step failed: {G.strerror(verr)}, losses {vlosses}", file=sys.stderr)
        sys.exit(1)
    # Mixed precision (bf16 matmul operands; fp32 master weights, AdamW and every other
    # operation) at the same shape: 2 warm-up steps (the second with events on every
    # kernel), 5 timed steps.
    bm = G.GPT2(w.model, w.B, w.T, stream=stream, variant=G.VARIANT_BF16)
    bm.params.copy_(model.params)
    tb = 0

    def bstep():
        nonlocal tb
        tb += 1
        loss = bm.forward(tx, ty)
        bm.zero_grad()
        bm.backward_update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, tb)
        return loss

    bstep()
    bm.profile_enable(True)
    bstep()
    torch.cuda.synchronize()
    bkernels = bm.profile_entries()
    bm.profile_enable(False)
    t4 = time.perf_counter()
    blosses = [bstep() for _ in range(5)]
    torch.cuda.synchronize()
    dt_bf = (time.perf_counter() - t4) / 5
    berr = bm.last_error()
    bm.close()
    if berr != 0 or not all(np.isfinite(blosses)):
        print(f"bench: mixed-precision step failed: {G.strerror(berr)}, losses {blosses}", file=sys.stderr)
        sys.exit(1)
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
    out["ms_per_step_without_events"] = dt_plain * 1e3 / args.steps
    out["roofline"] = roofline(kernels)
    # The same kernel measured alone (single-stream step): in the timed schedule its
    # launches overlap the main chain's kernels, so their durations include shared CUs.
    iso = [e for e in isolated if e["name"] == out["roofline"]["kernel"]]
    if iso:
        r = roofline(iso)
        out["roofline"]["isolated"] = {k: r[k] for k in ("achieved", "frac", "avg_launch_us", "launches")}
    out["roofline"]["schedule"] = ("timed steps overlap each layer's weight-gradient GEMMs (second stream) "
                                   "with the dgrad/attention/LayerNorm chain; 'isolated' is one "
                                   "single-stream step")
    out["generation"] = {
        "new_tokens": gen_new, "prompt": [eot], "tokens_per_s": gen_new / dt_gen,
        "ms_per_token": dt_gen * 1e3 / gen_new, "batch": 1,
        "method": "forward over the whole prefix per token (no key/value cache), then sample_mult on the "
                  "last position; coins from numpy default_rng(7)",
        "sample_kernel_us": sk[0]["ms"] * 1e3 / sk[0]["launches"] if sk else None,
        "first_tokens": [int(v) for v in gen[:9]],
    }
    vb = {k["name"]: k for k in breakdown(vkernels, 1)}
    out["variant_rmsnorm_rope"] = {
        "tokens_per_s": tokens / dt_var, "ms_per_step": dt_var * 1e3, "steps": 5,
        "what": "every LayerNorm replaced by RMSNorm, rotary q/k positions instead of wpe; same shape and step",
        "kernels": {n: vb[n] for n in ("rope_kernel<1>", "rope_kernel<-1>", "rms_fwd_kernel", "rms_bwd_kernel")
                    if n in vb},
    }
    bf_gemms = [k for k in bkernels if k["name"].startswith("gemm_bf16_kernel")]
    out["mixed_precision_bf16"] = {
        "tokens_per_s": tokens / dt_bf, "ms_per_step": dt_bf * 1e3, "steps": 5,
        "loss_first_last": [blosses[0], blosses[-1]],
        "what": "every linear layer and the LM head multiply bf16 roundings of their operands on the bf16 "
                "matrix cores (fp32 sums); fp32 master weights, AdamW, LayerNorm, attention, softmax/CE",
        "roofline_bf16_gemm": roofline(bf_gemms) if bf_gemms else None,
        "kernels": breakdown(bkernels, 1)[:16],
    }
    out["kernels"] = breakdown(all_kernels, max(1, args.warmup - 1))
    out["kernels_isolated"] = breakdown(isolated, 1)
    traffic = recorded_traffic(out["roofline"]["kernel"])
    if traffic is not None:
        out["roofline"]["traffic"] = traffic
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 2 * 4 * n
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
