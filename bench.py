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
plus the same kernel in a single-stream step), the aggregate matrix-core and HBM
fractions of the kernel classes, the chip's measured ceilings at its running clock
(matrix-core and copy probes), the standalone LayerNorm workload (8192 x 768) over
rotating buffers larger than the last-level cache, and the CPU oracle timed on a bounded
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


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the JSON result)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)

PEAK_FP32_MFMA = 157.3e12
PEAK_BF16_MFMA = 2.5e15  # dense
PEAK_HBM = 8.0e12


def mfma_peak(name: str) -> float:
    """Matrix-core peak of a kernel's operand type: the mixed-precision kernels (GEMMs and
    attention, every name with _bf16) multiply bf16, every other kernel fp32."""
    return PEAK_BF16_MFMA if "_bf16" in name else PEAK_FP32_MFMA


def aggregates(kernels):
    """Aggregate fractions over one step's kernels: the GEMMs' and the attention kernels'
    summed algorithmic flops over their summed time against the matrix-core peak of their
    type, and the memory-bound kernels' summed algorithmic bytes over their summed time
    against HBM."""
    def frac_mfma(ks):
        if not ks:
            return None
        fl = sum(k["flops"] for k in ks)
        ms = sum(k["ms"] for k in ks)
        peak = mfma_peak(ks[0]["name"])
        return dict(kernels=len(ks), ms=ms, tflops=fl / (ms / 1e3) / 1e12, frac=fl / (ms / 1e3) / peak)
    gemm = [k for k in kernels if k["flops"] > 0 and k["name"].startswith("gemm")]
    attn = [k for k in kernels if k["flops"] > 0 and k["name"].startswith("attn")]
    mem = [k for k in kernels if k["flops"] == 0 and k["bytes"] > 0]
    ms_mem = sum(k["ms"] for k in mem)
    by = sum(k["bytes"] for k in mem)
    return dict(gemm=frac_mfma(gemm), attention=frac_mfma(attn),
                memory=dict(kernels=len(mem), ms=ms_mem, gbps=by / (ms_mem / 1e3) / 1e9,
                            frac=by / (ms_mem / 1e3) / PEAK_HBM) if mem else None)


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
        e = dict(name=k["name"], ms_per_step=k["ms"] / steps, launches_per_step=k["launches"] / steps,
                 alg_flops_per_launch=k["flops"] / k["launches"], alg_bytes_per_launch=k["bytes"] / k["launches"])
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


def physical_cores() -> int:
    """Physical cores of the host (distinct core/socket pairs lscpu lists)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu", "-p=CORE,SOCKET"], capture_output=True, text=True, check=True).stdout
        pairs = {l for l in out.splitlines() if l and not l.startswith("#")}
        return len(pairs) or (os.cpu_count() or 1)
    except (OSError, subprocess.CalledProcessError):
        return os.cpu_count() or 1


def cpu_baseline(w: S.Workload, timed: int = 2):
    """The oracle as it stands, float32, built for this host (-march=native), on a bounded
    sample of the workload: one of its B sequences (1/B of the batch, T tokens), one
    warm-up step and `timed` timed full steps (forward, zero_grad, backward, AdamW) with
    as many threads as the host has physical cores available to this process, then one
    timed step at 8 threads (the pages' OMP_NUM_THREADS=8)."""
    from oracle import build as OB
    from oracle import oracle as O
    OB.build_native("f32")
    prec = "f32_native"
    params = S.init_params(w.model)
    x, y = S.tokens(w)
    x, y = x[:1], y[:1]
    phys = physical_cores()
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    env = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(phys, avail, env) if env > 0 else min(phys, avail)
    m = O.OracleGPT2(w.model, 1, w.T, params, prec)

    def one(t):
        t0 = time.perf_counter()
        m.forward(x, y)
        m.zero_grad()
        m.backward()
        m.update(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
        return time.perf_counter() - t0

    O.set_threads(threads, prec)
    warm = one(1)
    times = [one(2 + i) for i in range(timed)]
    O.set_threads(8, prec)
    t8 = one(2 + timed)
    used = O.load(prec).oracle_get_threads()
    O.set_threads(threads, prec)
    m.close()
    med = float(np.median(times))
    flops = step_flops(w.model, 1, w.T)
    return dict(value=w.T / med, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"1 of the {w.B} sequences ({w.T} tokens, 1/{w.B} of the batch) of the same workload; "
                       f"float32 oracle built -march=native; 1 warm-up step ({warm:.1f} s) then {timed} timed "
                       f"full steps (forward, zero_grad, backward, AdamW), median {med:.2f} s",
                host_physical_cores=phys, cpus_available=avail, threads=threads,
                tflops=flops / med / 1e12, step_s=[round(v, 3) for v in times],
                omp8=dict(threads=used, step_s=round(t8, 3), tokens_per_s=w.T / t8),
                pages_context="the pages' plain C step on an Apple M3 Max with OMP_NUM_THREADS=8: 1.29-1.45 s "
                              "per step of 256 tokens (GPT-2 124M, B=4, T=64), about 176-199 tokens/s")


def layernorm_standalone(G, torch, rounds: int = 5, sets: int = 8):
    """The standalone LayerNorm workload (8192 x 768, eps 1e-5) through the C ABI, over
    `sets` rotating buffer sets (x, dy, y, dx: 100 MB each, 805 MB in all, beyond the
    last-level cache), timed with HIP events on the stream the calls run on: per round,
    the sets' forwards back to back between one event pair, then their backwards; the
    median round over the set count."""
    N, C = S.LAYERNORM_ROWS, S.LAYERNORM_C
    x, gw, gb, dy = S.layernorm_inputs()
    st = torch.cuda.current_stream()
    bufs = []
    for i in range(sets):
        tx = torch.from_numpy(x).cuda().roll(i, 0).contiguous()
        bufs.append(dict(x=tx, dy=torch.from_numpy(dy).cuda().roll(i, 0).contiguous(),
                         y=torch.empty_like(tx), dx=torch.empty_like(tx),
                         mean=torch.empty(N, device="cuda"), rstd=torch.empty(N, device="cuda")))
    tw, tb = torch.from_numpy(gw).cuda(), torch.from_numpy(gb).cuda()
    dw, db = torch.empty_like(tw), torch.empty_like(tb)
    ws = torch.empty(max(1, G.layernorm_backward_workspace(N, C)), device="cuda")
    # each round: the 8 sets' forwards back to back between one event pair, then their
    # backwards (one event pair per batch keeps the events' own cost out of the average)
    fwd, bwd = [], []
    for r in range(rounds + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(st)
        for b in bufs:
            G.layernorm_forward(b["y"], b["mean"], b["rstd"], b["x"], tw, tb, 1e-5, stream=st)
        e[1].record(st)
        for b in bufs:
            G.layernorm_backward(b["dx"], dw, db, b["dy"], b["x"], tw, b["mean"], b["rstd"], ws, stream=st)
        e[2].record(st)
        if r:
            fwd.append(e[:2])
            bwd.append(e[1:])
    torch.cuda.synchronize()
    tf = float(np.median([a.elapsed_time(b) for a, b in fwd])) / 1e3 / sets
    tbw = float(np.median([a.elapsed_time(b) for a, b in bwd])) / 1e3 / sets
    # algorithmic bytes: forward reads x, writes y, mean and rstd (and reads w, b);
    # backward reads dy, x, mean, rstd (and w), writes dx, dw and db
    bf = 4.0 * (2 * N * C + 2 * N + 2 * C)
    bb = 4.0 * (3 * N * C + 2 * N + 3 * C)
    return dict(shape=[N, C], buffer_sets=sets, bytes_all_sets=sets * 4 * 4 * N * C,
                forward=dict(us=tf * 1e6, gbps=bf / tf / 1e9, frac_hbm=bf / tf / PEAK_HBM),
                backward=dict(us=tbw * 1e6, gbps=bb / tbw / 1e9, frac_hbm=bb / tbw / PEAK_HBM,
                              note="both kernels of the call (per-row pass and the dgamma/dbeta reduction)"))


def ceilings(G, torch):
    """The chip's ceilings at its running clock: matrix-core probes (fp32 16x16x4 and
    bf16 16x16x32 products in registers, no memory traffic) and a 1 GiB float4 copy."""
    st = torch.cuda.current_stream()
    out = torch.empty(G.probe_mfma_out_floats(), device="cuda")
    res = {}
    for kind, name, peak, iters in ((0, "fp32_mfma", PEAK_FP32_MFMA, 6000), (1, "bf16_mfma", PEAK_BF16_MFMA, 3000)):
        best = None
        for blocks in (512, 1024):  # two or four waves per SIMD
            G.probe_mfma(kind, 100, out, blocks=blocks, stream=st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fl = G.probe_mfma(kind, iters * 1024 // blocks, out, blocks=blocks, stream=st)
            e1.record(st)
            torch.cuda.synchronize()
            s = e0.elapsed_time(e1) / 1e3
            if best is None or fl / s > best[0]:
                best = (fl / s, blocks)
        res[name] = dict(tflops=best[0] / 1e12, frac_of_datasheet=best[0] / peak, waves_per_simd=best[1] // 256)
    n = (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    G.probe_copy(dst, src, stream=st)
    best = None
    for blocks in (1024, 2048, 4096, 8192, 16384):
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            G.probe_copy(dst, src, blocks=blocks, stream=st)
            e1.record(st)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        s = min(a.elapsed_time(b) for a, b in ts) / 1e3
        if best is None or s < best[0]:
            best = (s, blocks)
    s = best[0]
    res["copy_1gib"] = dict(gbps=2.0 * 4 * n / s / 1e9, frac_of_datasheet=2.0 * 4 * n / s / PEAK_HBM, blocks=best[1])
    # the platform's own device-to-device copy of the same buffers, for comparison
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        dst.copy_(src)
        e1.record(st)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    s = min(a.elapsed_time(b) for a, b in ts) / 1e3
    res["platform_copy_1gib"] = dict(gbps=2.0 * 4 * n / s / 1e9, frac_of_datasheet=2.0 * 4 * n / s / PEAK_HBM)
    del src, dst
    res["note"] = "fractions elsewhere in this line use the datasheet peaks (fp32 157.3 TFLOP/s, bf16 2.5 PFLOP/s, HBM 8 TB/s)"
    return res


def same_size_copies(G, torch, entries, stream):
    """For each memory-bound kernel of a breakdown (1 MB or more per launch): the time of a
    plain float4 copy (the library's probe copy) that reads and writes the kernel's
    algorithmic bytes per launch in equal halves, timed the same way (one event pair
    around one launch, best grid of several, best of five launches).  Short launches pay
    their ramp, drain and event cost whatever they compute, so this is the ceiling a
    kernel of that size can reach here; the ratio says how close each kernel comes."""
    out = {}
    for e in entries:
        if "gbps" not in e or e["gbps"] <= 0:
            continue
        us = e["ms_per_step"] * 1e3 / e["launches_per_step"]
        nbytes = e["gbps"] * 1e9 * us / 1e6
        if nbytes < 1e6:
            continue
        n = max(4096, int(nbytes / 8) // 4 * 4)
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        G.probe_copy(dst, src, blocks=256, stream=stream)
        best = None
        for blocks in (256, 512, 1024, 2048, 4096):
            blocks = min(blocks, max(1, n // (4 * 1024)))
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                G.probe_copy(dst, src, blocks=blocks, stream=stream)
                e1.record(stream)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            t = min(a.elapsed_time(b) for a, b in ts) * 1e3
            if best is None or t < best:
                best = t
        del src, dst
        out[e["name"]] = dict(bytes_per_launch=8 * n, kernel_us=us, copy_us=best,
                              copy_frac_hbm=8 * n / (best / 1e6) / PEAK_HBM, kernel_vs_copy=best / us)
    return out


def variant_leg(G, torch, w, stream, params, tx, ty, variant, steps=5):
    """A second model of the same shape in another variant, from the same parameters:
    2 warm-up steps (the second with events on every kernel), `steps` timed steps."""
    vm = G.GPT2(w.model, w.B, w.T, stream=stream, variant=variant)
    vm.params.copy_(params)
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
    kernels = vm.profile_entries()
    vm.profile_enable(False)
    t0 = time.perf_counter()
    losses = [vstep() for _ in range(steps)]
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    err = vm.last_error()
    vm.close()
    if err != 0 or not all(np.isfinite(losses)):
        print(f"bench: variant {variant} step failed: {G.strerror(err)}, losses {losses}", file=sys.stderr)
        sys.exit(1)
    return kernels, dt, losses


def generation_leg(model, w, torch):
    """Forward-only generation with the model's current weights (the pages' sample loop):
    64 new tokens from the end-of-text token, one fixed coin per token, each step
    recomputing the whole prefix; the sampling kernel timed with events."""
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
    return {
        "new_tokens": gen_new, "prompt": [eot], "tokens_per_s": gen_new / dt_gen,
        "ms_per_token": dt_gen * 1e3 / gen_new, "batch": 1,
        "method": "forward over the whole prefix per token (no key/value cache), then sample_mult on the "
                  "last position; coins from numpy default_rng(7)",
        "sample_kernel_us": sk[0]["ms"] * 1e3 / sk[0]["launches"] if sk else None,
        "first_tokens": [int(v) for v in gen[:9]],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=S.GPT2_124M.name)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="only the training step (for profiler runs): no generation, variants, standalone "
                         "LayerNorm, ceilings or CPU baseline")
    ap.add_argument("--variant", choices=("fp32", "bf16"), default="fp32",
                    help="variant of the timed step (bf16: the mixed-precision model; for profiler runs)")
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
    main_variant = G.VARIANT_BF16 if args.variant == "bf16" else 0
    model = G.GPT2(w.model, w.B, w.T, stream=stream, variant=main_variant)
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

    progress(f"{w.name}: warm-up")
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
    # only, recorded on the stream that launch runs on; one event pair per step on the
    # model's stream gives each step's time (median and spread).
    progress(f"timed steps ({args.steps})")
    model.profile_enable(True)
    model.profile_filter(dominant)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    losses = []
    for i in range(args.steps):
        step_ev[i].record(stream)
        losses.append(step())
    step_ev[-1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in zip(step_ev[:-1], step_ev[1:])]
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
        "dtype": "f32" if not main_variant else "bf16 matmul operands, f32 otherwise",
        "data": "synthetic (Zipf(1.1) int32 tokens with separator 50256 every 256; N(0,0.02) init)",
        "config": {"workload": w.name, "global_batch": w.B, "seq_len": w.T,
                   "layers": w.model.num_layers, "channels": w.model.channels,
                   "heads": w.model.num_heads, "vocab": w.model.vocab_size,
                   "parallelism": "single GPU"},
        "tflops": flops / (dt / args.steps) / 1e12,
        "step_roofline_frac": flops / PEAK_FP32_MFMA / (dt / args.steps),
        "loss_first_last": [losses[0], losses[-1]],
    }
    out["ms_per_step_median"] = float(np.median(step_ms))
    out["tokens_per_s_at_median"] = tokens / (out["ms_per_step_median"] / 1e3)
    out["ms_per_step_min_max"] = [min(step_ms), max(step_ms)]
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
    out["kernels"] = breakdown(all_kernels, max(1, args.warmup - 1))
    out["kernels_isolated"] = breakdown(isolated, 1)
    # Each memory-bound kernel against a plain copy of its own bytes per launch (not in
    # profiler runs, whose only probe copies are the calibration copies).
    if not args.step_only:
        out["memory_kernels_vs_same_size_copy"] = same_size_copies(G, torch, out["kernels_isolated"], stream)
    # Aggregate fractions from the single-stream step, where kernel times do not overlap.
    out["aggregates_isolated"] = aggregates(isolated)
    out["aggregates_isolated"]["note"] = ("GEMM and attention: summed algorithmic flops over summed kernel "
                                          "time vs the matrix-core peak of their type; memory: summed "
                                          "algorithmic bytes of the memory-bound kernels over their summed "
                                          "time vs 8 TB/s")
    traffic = recorded_traffic(out["roofline"]["kernel"])
    if traffic is not None:
        out["roofline"]["traffic"] = traffic
    if not args.step_only:
        progress("generation")
        out["generation"] = generation_leg(model, w, torch)
        if not main_variant:
            progress("RMSNorm + RoPE variant")
            vkernels, dt_var, _ = variant_leg(G, torch, w, stream, model.params, tx, ty,
                                              G.VARIANT_RMSNORM | G.VARIANT_ROPE)
            vb = {k["name"]: k for k in breakdown(vkernels, 1)}
            out["variant_rmsnorm_rope"] = {
                "tokens_per_s": tokens / dt_var, "ms_per_step": dt_var * 1e3, "steps": 5,
                "what": "every LayerNorm replaced by RMSNorm, rotary q/k positions instead of wpe; same shape "
                        "and step",
                "kernels": {n: vb[n] for n in ("rope_kernel<1>", "rope_kernel<-1>", "rms_fwd_kernel",
                                               "rms_bwd_kernel") if n in vb},
            }
            progress("mixed-precision variant")
            bkernels, dt_bf, blosses = variant_leg(G, torch, w, stream, model.params, tx, ty, G.VARIANT_BF16)
            bf_gemms = [k for k in bkernels if k["name"].startswith("gemm_bf16")]
            out["mixed_precision_bf16"] = {
                "tokens_per_s": tokens / dt_bf, "ms_per_step": dt_bf * 1e3, "steps": 5,
                "loss_first_last": [blosses[0], blosses[-1]],
                "what": "every linear layer and the LM head multiply bf16 roundings of their operands on the "
                        "bf16 matrix cores (fp32 sums); fp32 master weights, AdamW, LayerNorm, attention, "
                        "softmax/CE",
                "roofline_bf16_gemm": roofline(bf_gemms) if bf_gemms else None,
                "aggregates": aggregates(bkernels),
                "kernels": breakdown(bkernels, 1)[:16],
            }
        progress("standalone LayerNorm and ceilings")
        out["layernorm_standalone"] = layernorm_standalone(G, torch)
        out["ceilings"] = ceilings(G, torch)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            G.probe_copy(dst, src, blocks=4096, stream=stream)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 2 * 4 * n
    if not args.no_cpu_baseline and not args.step_only:
        progress("CPU baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
