#!/usr/bin/env python3
"""Benchmark of the NF4 QLoRA linear hot path on one MI355X.

One step = the whole path over one batch of the Llama-7B-shaped MLP workload
(gate and up 4096->11008, down 11008->4096; M = 4096 tokens = batch 4 x seq
1024; LoRA rank 64, alpha 16; weights fp32 N(0, 0.02^2), NF4 + double
quantization): for each of the three linears, the fused dequant-GEMM forward
(saving T) and the backward (dX, dA, dB).  The frozen weights are quantized
once, before the timed region (a training step does not re-quantize them);
the step with the three quantizations included is reported beside it.
Inputs are seeded synthetic data resident in HBM before the timed region.
Before the W warmup steps, steps run untimed for --settle seconds (0.5): the
GPU idles while the host draws the inputs, and its clocks take tens of
milliseconds to come back up.  The JSON line carries the min / median / max
of the K timed steps (events at every step boundary).

value = fwd+bwd algorithmic FLOP per step / step time.  Algorithmic FLOP per
linear: 4*M*N*K + 6*M*r*(K+N).

Extra objects on the JSON line:
  roofline       the dominant kernel (by time per step), measured live with
                 HIP events attached to its launches in the last timed step;
                 frac against the 2.5 PFLOP/s dense bf16 spec, and beside it
                 against the in-run MFMA loop (measured_peaks);
  measured_peaks a register-only v_mfma_f32_16x16x32_bf16 loop on every SIMD
                 (the MFMA rate the chip sustains) and a streaming copy of
                 1 GiB (the HBM rate of a plain read + write), both from the
                 library; torch's bf16 matmul on the 7B MLP shape as context;
  workloads      the same fwd+bwd step on the 7B decoder block (seven
                 linears, M = 8192) and the 65B layer (seven linears, M =
                 2048), each with its dominant kernel's roofline;
  m_sweep        the gate linear (11008x4096, r = 64) at M = 1, 16, 17, 64,
                 128, 512 (one 8-way data-parallel shard of the 4096-token
                 batch) and 4096: forward and forward+backward time;
  gemv           the q_proj forward (4096x4096, r = 16) at M = 1 and 16: the
                 whole forward (T partials + dequant-GEMV) per call when 64
                 forwards over 64 quantized copies (~0.55 GB, more than twice
                 the 256 MB last-level cache) are captured in one graph and
                 replayed, against the forward's algorithmic bytes (codes,
                 constants, X, A, B, Y); the GEMV kernel's own event-timed
                 median beside it;
  bulk_quantize  NF4 + double quantization throughput over streamed bf16
                 weights (the 7B-block and 65B-layer tensor lists: 6.7B and
                 65B parameters); only the quantize kernels are timed;
  adamw, merge, formats, f16_step   the next rows (AdamW step, LoRA merge,
                 comparison formats, fp16 compute);
  cpu_baseline   the oracle (numpy, fp64) on a bounded sample: one whole step
                 of the 7B MLP workload; breadth: quantize params/s on
                 several shapes and fp64 fwd+bwd of one linear of each
                 workload.

roofline.traffic is the HBM traffic (bytes per launch) of the dominant kernel
as rocprofv3's FETCH_SIZE and WRITE_SIZE counters read it, scaled by what the
same counters read for the library's streaming copy of known size
(--copy-calibration).  It is taken from the summary under profiles/ and
reported only while the kernel's sources are byte-identical to the ones
profiled; otherwise null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--no-cpu-baseline]
                       [--no-gemv] [--no-adamw] [--no-merge] [--no-formats] [--no-f16]
                       [--no-workloads] [--no-sweep] [--no-bulk] [--bulk-sample]
"""

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QLoRA NF4 linear fwd+bwd TFLOP/s @7B MLP M=4096; dequant-GEMV GB/s @M=1"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each GEMM kernel is compiled from (its traffic figure is tied to them).
KERNEL_SOURCES = {
    "fwd_gemm_kernel": ("fwd.hip", "common.h", "tiling.h"),
    "dx_gemm_kernel": ("dx.hip", "common.h", "tiling.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic_mlp7b.txt")


def _code_only(text):
    """The source without comments and blank space, so that edits of comments
    do not count as changes of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "quantized_fine_tuning_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def profiled_traffic(kernel):
    """Copy-calibrated FETCH_SIZE + WRITE_SIZE bytes per launch of `kernel`
    from the committed counter summary, or None when the summary is missing or
    was taken on other sources."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    rec, cur = {}, None
    for ln in lines:
        parts = ln.split()
        if len(parts) != 2 or ln.startswith("#"):
            continue
        if parts[0] == "kernel":
            cur = rec.setdefault(parts[1], {})
        elif cur is not None:
            cur[parts[0]] = parts[1]
    r = rec.get(kernel)
    if not r or r.get("sources_sha256") != kernel_source_digest(kernel):
        return None
    return int(r["fetch_bytes_per_launch"]) + int(r["write_bytes_per_launch"])


def linear_flops(M, N, K, r):
    return 4 * M * N * K + 6 * M * r * (K + N)


def gemv_forward_bytes(M, N, K, r):
    """Bytes the whole M <= 16 forward must move (the algorithmic count):
    packed codes, e4m3 constants, group scales, mean, X, A and B in; Y (bf16)
    out.  8,933,380 bytes for the q_proj weight at M = 1, r = 16."""
    nb = N * K // 64
    ng = (nb + 255) // 256
    return N * K // 2 + nb + 4 * ng + 4 + 2 * M * K + 2 * r * (K + N) + 2 * M * N


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def timed_events(torch, n):
    evs = []
    s = torch.cuda.current_stream()
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)  # materialise the underlying HIP events
        b.record(s)
        evs.append((a, b))
    return evs


def make_layers(torch, q, widx, M, f16=False, device_inputs=False):
    """Inputs of one workload on the device, weights quantized once."""
    from workloads import Inputs, device_normal

    cvt = (lambda x: x.to(torch.float16)) if f16 else (lambda x: x)  # noqa: E731
    w = Inputs(widx)
    r = w.w.rank
    layers = []
    for li, (name, N, K) in enumerate(w.w.layers):
        t0 = time.time()
        L = {"name": name, "N": N, "K": K}
        seed = 1000 * widx + 10 * li
        if device_inputs:
            Wd = device_normal(torch, (N, K), seed, 0.02)
            L["X"] = cvt(device_normal(torch, (M, K), seed + 1))
            L["dY"] = cvt(device_normal(torch, (M, N), seed + 2))
            L["A"] = cvt(device_normal(torch, (r, K), seed + 3, 0.02))
            L["B"] = cvt(device_normal(torch, (N, r), seed + 4, 0.01))
        else:
            Wd = torch.from_numpy(w.weight(li)).cuda()
            L["X"] = cvt(dev_bf16(torch, w.X(li, M)))
            L["dY"] = cvt(dev_bf16(torch, w.dY(li, M)))
            L["A"] = cvt(dev_bf16(torch, w.lora_A(li)))
            L["B"] = cvt(dev_bf16(torch, w.lora_B(li)))
        sz = q.qlora_nf4_sizes(N, K, M, r)
        L["W"] = Wd
        L["qt"] = q.Nf4Tensor.empty(N, K)
        L["wsq"] = q.workspace(sz["quantize_ws_bytes"])
        q.qlora_nf4_quantize(Wd, L["qt"], L["wsq"])
        L["wsf"] = q.workspace(sz["fwd_ws_bytes"])
        L["wsb"] = q.workspace(sz["bwd_ws_bytes"])
        dt16 = torch.float16 if f16 else torch.bfloat16
        L["Y"] = torch.empty(M, N, dtype=dt16, device="cuda")
        L["T"] = torch.empty(M, r, dtype=torch.float32, device="cuda")
        L["dX"] = torch.empty(M, K, dtype=dt16, device="cuda")
        L["dA"] = torch.empty(r, K, dtype=torch.float32, device="cuda")
        L["dB"] = torch.empty(N, r, dtype=torch.float32, device="cuda")
        layers.append(L)
        log(f"[bench] inputs of workload {widx} {name} {N}x{K} M={M} ready ({time.time() - t0:.1f}s)")
    return w, layers


def run_step(torch, q, args, widx=3, M=None, f16=False, steps=None, warmup=None, device_inputs=False,
             with_quantize=True):
    """The timed fwd+bwd step of one workload; then the same step with the
    quantization of every weight included."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    from workloads import Inputs
    M = Inputs(widx).w.tokens[0] if M is None else M
    w, layers = make_layers(torch, q, widx, M, f16, device_inputs)
    r, alpha = w.w.rank, w.w.alpha

    kinds = ("quantize", "fwd_gemm", "dx_gemm")
    kid = {"quantize": q.QLORA_KERNEL_QUANTIZE, "fwd_gemm": q.QLORA_KERNEL_FWD_GEMM,
           "dx_gemm": q.QLORA_KERNEL_DX_GEMM}
    # Each launch timed with its own events costs ~10 us of idle GPU time
    # around it, so only the launches of the last timed step carry events.
    events = {k: timed_events(torch, len(layers)) for k in kinds}

    def step(i=None, quantize=False, last=None):
        for li, L in enumerate(layers):
            j = li if i == last else None
            if quantize:
                if j is not None:
                    q.qlora_time_next_launch(kid["quantize"], *events["quantize"][j])
                q.qlora_nf4_quantize(L["W"], L["qt"], L["wsq"])
            if j is not None:
                q.qlora_time_next_launch(kid["fwd_gemm"], *events["fwd_gemm"][j])
            q.qlora_linear_fwd(L["qt"], L["X"], L["A"], L["B"], r, alpha, L["Y"], L["T"], L["wsf"])
            if j is not None:
                q.qlora_time_next_launch(kid["dx_gemm"], *events["dx_gemm"][j])
            q.qlora_linear_bwd(L["qt"], L["X"], L["dY"], L["A"], L["B"], r, alpha, L["T"],
                               L["dX"], L["dA"], L["dB"], L["wsb"])

    step_ms = []

    def timed(quantize, n, nw):
        # The clocks ramp up over tens of milliseconds once the GPU is busy
        # again (it idles while the host draws the inputs): steps are run
        # for args.settle seconds first, then the warmup steps, then the
        # timed ones, with an event at every step boundary.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle:
            step(quantize=quantize)
            torch.cuda.synchronize()
        for _ in range(nw):
            step(quantize=quantize)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            step(i, quantize, last=n - 1)
            ev[i + 1].record()
        torch.cuda.synchronize()
        step_ms[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        return ev[0].elapsed_time(ev[n]) / n

    ms_per_step = timed(False, steps, warmup)
    step_stats = {"min": round(min(step_ms), 4), "median": round(statistics.median(step_ms), 4),
                  "max": round(max(step_ms), 4)}
    log(f"[bench] workload {widx}: {steps} timed fwd+bwd steps: {ms_per_step:.3f} ms/step "
        f"(per step {step_stats})")
    per_kernel = {}
    for k in ("fwd_gemm", "dx_gemm"):
        durs = [a.elapsed_time(b) for a, b in events[k]]
        per_kernel[k] = {"avg_ms": statistics.mean(durs), "total_ms_per_step": sum(durs),
                         "launches_per_step": len(layers)}
    ms_q = None
    if with_quantize:
        ms_q = timed(True, max(2, steps // 4), 1)
        durs = [a.elapsed_time(b) for a, b in events["quantize"]]
        per_kernel["quantize"] = {"avg_ms": statistics.mean(durs), "total_ms_per_step": sum(durs),
                                  "launches_per_step": len(layers)}
        q_bytes = statistics.mean(L["N"] * L["K"] * ((4 if L["W"].dtype == torch.float32 else 2) + 0.5 + 1 / 64)
                                  + 4 * (L["N"] * L["K"] // 16384) + 4 for L in layers)
        per_kernel["quantize"]["gbs"] = q_bytes / (per_kernel["quantize"]["avg_ms"] * 1e-3) / 1e9
        log(f"[bench] workload {widx}: step with the quantization of every weight: {ms_q:.3f} ms")

    flops = sum(linear_flops(M, L["N"], L["K"], r) for L in layers)
    # algorithmic work per launch, averaged over the step's launches of each kernel
    fwd_flop = statistics.mean(2 * M * L["N"] * L["K"] + 2 * M * L["N"] * r for L in layers)
    dx_flop = statistics.mean(2 * M * L["N"] * L["K"] + 2 * M * L["K"] * r for L in layers)
    per_kernel["fwd_gemm"]["tflops"] = fwd_flop / (per_kernel["fwd_gemm"]["avg_ms"] * 1e-3) / 1e12
    per_kernel["dx_gemm"]["tflops"] = dx_flop / (per_kernel["dx_gemm"]["avg_ms"] * 1e-3) / 1e12
    dom = max(("fwd_gemm", "dx_gemm"), key=lambda k: per_kernel[k]["total_ms_per_step"])
    ach = per_kernel[dom]["tflops"]
    kname = {"fwd_gemm": "fwd_gemm_kernel", "dx_gemm": "dx_gemm_kernel"}[dom]
    roofline = {"bound": "mfma", "kernel": kname,
                "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": profiled_traffic(kname) if widx == 3 and not f16 else None,
                "avg_launch_ms": round(per_kernel[dom]["avg_ms"], 4),
                "flop_per_launch": int(fwd_flop if dom == "fwd_gemm" else dx_flop)}
    del layers
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "step_ms": step_stats, "ms_per_step_with_quantize": ms_q,
            "flops": flops, "M": M, "r": r,
            "alpha": alpha, "layers": [list(x) for x in w.w.layers], "per_kernel": per_kernel,
            "roofline": roofline}


def run_workloads(torch, q, args):
    """fwd+bwd of the 7B decoder block (M = 8192) and the 65B layer (M = 2048)."""
    out = {}
    for widx, name in ((4, "llama-7b decoder block, 7 linears"), (5, "65b-shaped layer, 7 linears")):
        res = run_step(torch, q, args, widx, steps=max(3, args.steps // 2), warmup=2, device_inputs=True,
                       with_quantize=False)
        tf = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
        rl = res["roofline"]
        out[f"workload{widx}"] = {"workload": name, "tokens": res["M"], "lora_rank": res["r"],
                                  "flop_per_step": res["flops"], "ms_per_step": round(res["ms_per_step"], 4),
                                  "step_ms": res["step_ms"],
                                  "TFLOP/s": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "roofline": rl,
                                  "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                                                  for kk, vv in v.items()} for k, v in res["per_kernel"].items()}}
        log(f"[bench] workload {widx}: {tf:.1f} TFLOP/s fwd+bwd")
    return out


def run_m_sweep(torch, q, args):
    """The gate linear (11008x4096, r = 64) at several token counts."""
    from workloads import device_normal

    N, K, r, alpha = 11008, 4096, 64, 16.0
    Wd = device_normal(torch, (N, K), 77, 0.02, bf16=False)
    qt = q.Nf4Tensor.empty(N, K)
    q.qlora_nf4_quantize(Wd, qt, q.workspace(q.qlora_nf4_sizes(N, K, 0, r)["quantize_ws_bytes"]))
    del Wd
    A = device_normal(torch, (r, K), 78, 0.02)
    B = device_normal(torch, (N, r), 79, 0.01)
    out = {}
    for M in (1, 16, 17, 64, 128, 512, 4096):
        X = device_normal(torch, (M, K), 80 + M)
        dY = device_normal(torch, (M, N), 81 + M)
        sz = q.qlora_nf4_sizes(N, K, M, r)
        wsf, wsb = q.workspace(sz["fwd_ws_bytes"]), q.workspace(sz["bwd_ws_bytes"])
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        T = torch.empty(M, r, dtype=torch.float32, device="cuda")
        dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dA = torch.empty(r, K, dtype=torch.float32, device="cuda")
        dB = torch.empty(N, r, dtype=torch.float32, device="cuda")

        def fwd():
            q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y, T, wsf)

        def bwd():
            q.qlora_linear_bwd(qt, X, dY, A, B, r, alpha, T, dX, dA, dB, wsb)

        n = 20
        for _ in range(3):
            fwd()
            bwd()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(n):
            fwd()
        e[1].record()
        for _ in range(n):
            fwd()
            bwd()
        e[2].record()
        torch.cuda.synchronize()
        f_ms = e[0].elapsed_time(e[1]) / n
        fb_ms = e[1].elapsed_time(e[2]) / n
        fl = linear_flops(M, N, K, r)
        out[f"M{M}"] = {"fwd_ms": round(f_ms, 4), "fwd_bwd_ms": round(fb_ms, 4),
                        "fwd_bwd_TFLOP/s": round(fl / (fb_ms * 1e-3) / 1e12, 2),
                        "fwd_bwd_frac_of_peak": round(fl / (fb_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "path": "dequant-GEMV" if M <= 16 else "dequant-in-tile GEMM"}
        log(f"[bench] gate M={M}: fwd {f_ms * 1e3:.1f} us, fwd+bwd {fb_ms * 1e3:.1f} us")
    return out


def run_gemv(torch, q, args):
    from workloads import Inputs

    w = Inputs(2)
    N, K = w.shape(0)
    r, alpha = w.w.rank, w.w.alpha
    W = torch.from_numpy(w.weight(0)).cuda()
    sz = q.qlora_nf4_sizes(N, K, 16, r)
    wsq = q.workspace(sz["quantize_ws_bytes"])
    copies = []
    for _ in range(args.gemv_copies):
        qt = q.Nf4Tensor.empty(N, K)
        q.qlora_nf4_quantize(W, qt, wsq)
        copies.append(qt)
    del W
    A = dev_bf16(torch, w.lora_A(0))
    B = dev_bf16(torch, w.lora_B(0))
    wsf = q.workspace(sz["fwd_ws_bytes"])
    out = {}
    for M in (1, 16):
        X = dev_bf16(torch, w.X(0, M))
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        T = torch.empty(M, r, dtype=torch.float32, device="cuda")
        n = args.gemv_iters
        evs = timed_events(torch, n)
        for i in range(10):
            q.qlora_linear_fwd(copies[i % len(copies)], X, A, B, r, alpha, Y, T, wsf)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for i in range(n):
            q.qlora_time_next_launch(q.QLORA_KERNEL_GEMV, *evs[i])
            q.qlora_linear_fwd(copies[i % len(copies)], X, A, B, r, alpha, Y, T, wsf)
        c1.record()
        torch.cuda.synchronize()
        durs = sorted(a.elapsed_time(b) for a, b in evs)
        med = statistics.median(durs)
        nbytes = gemv_forward_bytes(M, N, K, r)
        out[f"M{M}"] = {"gemv_kernel_us_median": round(med * 1e3, 3),
                        "gemv_kernel_us_p10": round(durs[n // 10] * 1e3, 3),
                        "gemv_kernel_us_p90": round(durs[(9 * n) // 10] * 1e3, 3),
                        "eager_call_us_mean": round(c0.elapsed_time(c1) / n * 1e3, 3),
                        "forward_bytes": nbytes}
        # the same forwards captured in one graph (one per quantized copy) and
        # replayed: the launch-bound decode loop without per-call host work
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for qt in copies:
                q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y, T, wsf)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for qt in copies:
                q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y, T, wsf)
        g.replay()
        torch.cuda.synchronize()
        reps = 5
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        per = g0.elapsed_time(g1) / (reps * len(copies)) * 1e3
        gbs = nbytes / (per * 1e-6) / 1e9
        out[f"M{M}"]["forward_us"] = round(per, 3)
        out[f"M{M}"]["GB/s"] = round(gbs, 1)
        out[f"M{M}"]["frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
        del g
        log(f"[bench] GEMV M={M}: whole forward (graph-replayed) {per:.2f} us, {gbs:.0f} GB/s; "
            f"GEMV kernel {med * 1e3:.2f} us median (events)")
    out["gate_M1"] = run_gemv_gate(torch, q, args)
    return out


def run_gemv_gate(torch, q, args):
    """The M = 1 forward of the 7B gate linear (11008x4096, r = 64), graph-replayed
    over 16 quantized copies (0.36 GB, more than the last-level cache)."""
    from workloads import device_normal

    N, K, r, alpha = 11008, 4096, 64, 16.0
    Wd = device_normal(torch, (N, K), 77, 0.02, bf16=False)
    wsq = q.workspace(q.qlora_nf4_sizes(N, K, 0, r)["quantize_ws_bytes"])
    copies = []
    for _ in range(16):
        qt = q.Nf4Tensor.empty(N, K)
        q.qlora_nf4_quantize(Wd, qt, wsq)
        copies.append(qt)
    del Wd
    A = device_normal(torch, (r, K), 78, 0.02)
    B = device_normal(torch, (N, r), 79, 0.01)
    X = device_normal(torch, (1, K), 81)
    wsf = q.workspace(q.qlora_nf4_sizes(N, K, 1, r)["fwd_ws_bytes"])
    Y = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
    T = torch.empty(1, r, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for qt in copies:
            q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y, T, wsf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            for qt in copies:
                q.qlora_linear_fwd(qt, X, A, B, r, alpha, Y, T, wsf)
    g.replay()
    torch.cuda.synchronize()
    reps = 5
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(reps):
        g.replay()
    g1.record()
    torch.cuda.synchronize()
    per = g0.elapsed_time(g1) / (reps * 4 * len(copies)) * 1e3
    nbytes = gemv_forward_bytes(1, N, K, r)
    gbs = nbytes / (per * 1e-6) / 1e9
    del g
    log(f"[bench] GEMV gate 11008x4096 M=1: whole forward (graph-replayed) {per:.2f} us, {gbs:.0f} GB/s")
    return {"N": N, "K": K, "lora_rank": r, "forward_bytes": nbytes, "forward_us": round(per, 3),
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def adamw_bytes(n, param_bytes=2):
    """Bytes one AdamW step must move per parameter: the parameter, gradient
    and two fp32 moments read, the parameter and the moments written."""
    return n * (2 * param_bytes + 4 + 4 * 4)


def run_adamw(torch, q, args):
    """The AdamW step on bf16 LoRA parameters with fp32 moments, one launch per
    step: (a) the six LoRA matrices of the 7B MLP at r = 64 (2.9 M
    parameters); (b) 8 tensors of 16 M parameters (128 M, beyond the last-level
    cache).  Kernel time from events attached to the launch."""
    out = {}
    cases = {"mlp_lora_r64": [64 * 4096, 11008 * 64, 64 * 4096, 11008 * 64, 64 * 11008, 4096 * 64],
             "8x16M": [16 << 20] * 8}
    for name, sizes in cases.items():
        g = torch.Generator(device="cuda").manual_seed(7)
        ts = []
        for n in sizes:
            p = (torch.randn(n, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            ts.append((p, torch.randn(n, device="cuda", generator=g) * 0.1,
                       torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")))
        n_iter = 50
        evs = timed_events(torch, n_iter)
        for i in range(5):
            q.qlora_adamw_step(ts, 1e-4, 0.9, 0.999, 1e-8, 0.01, i + 1)
        torch.cuda.synchronize()
        for i in range(n_iter):
            q.qlora_time_next_launch(q.QLORA_KERNEL_ADAMW, *evs[i])
            q.qlora_adamw_step(ts, 1e-4, 0.9, 0.999, 1e-8, 0.01, i + 6)
        torch.cuda.synchronize()
        durs = sorted(a.elapsed_time(b) for a, b in evs)
        med = statistics.median(durs)
        nparams = sum(sizes)
        nbytes = adamw_bytes(nparams)
        gbs = nbytes / (med * 1e-3) / 1e9
        out[name] = {"params": nparams, "kernel_us_median": round(med * 1e3, 3),
                     "bytes": nbytes, "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench] AdamW {name}: {med * 1e3:.2f} us median, {gbs:.0f} GB/s")
        del ts
    return out


def merge_bytes(N, K, r):
    """Bytes the merge kernel must move: packed codes, e4m3 constants, group
    scales, mean, A and B in; the 16-bit merged weight out."""
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * r * K + 2 * N * r + 2 * N * K


def run_merge(torch, q, args):
    """The LoRA merge (bf16 output) of the 7B MLP's three weights at r = 64:
    median kernel time per weight from events attached to the launch; then,
    on the gate weight, what re-quantizing the merged weight costs in error."""
    from workloads import Inputs

    w = Inputs(3)
    r, alpha = w.w.rank, w.w.alpha
    out = {"layers": {}}
    for li, (name, N, K) in enumerate(w.w.layers):
        Wd = torch.from_numpy(w.weight(li)).cuda()
        qt = q.Nf4Tensor.empty(N, K)
        q.qlora_nf4_quantize(Wd, qt, q.workspace(q.qlora_nf4_sizes(N, K, 0, r)["quantize_ws_bytes"]))
        A, B = dev_bf16(torch, w.lora_A(li)), dev_bf16(torch, w.lora_B(li))
        Wm = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        n_iter = 30
        evs = timed_events(torch, n_iter)
        for _ in range(3):
            q.qlora_merge_lora(qt, A, B, r, alpha, Wm)
        torch.cuda.synchronize()
        for i in range(n_iter):
            q.qlora_time_next_launch(q.QLORA_KERNEL_MERGE, *evs[i])
            q.qlora_merge_lora(qt, A, B, r, alpha, Wm)
        torch.cuda.synchronize()
        med = statistics.median(a.elapsed_time(b) for a, b in evs)
        nbytes = merge_bytes(N, K, r)
        gbs = nbytes / (med * 1e-3) / 1e9
        out["layers"][name] = {"N": N, "K": K, "kernel_us_median": round(med * 1e3, 3), "bytes": nbytes,
                               "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench] merge {name} {N}x{K}: {med * 1e3:.2f} us median, {gbs:.0f} GB/s")
        if li == 0:
            # re-quantization of the merged weight (the error merging and
            # re-quantizing brings back); norms in fp64 on the device
            W_hat = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
            q.qlora_dequantize(qt, W_hat)
            qt2 = q.Nf4Tensor.empty(N, K)
            q.qlora_nf4_quantize(Wm, qt2, q.workspace(q.qlora_nf4_sizes(N, K, 0, r)["quantize_ws_bytes"]))
            back = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
            q.qlora_dequantize(qt2, back)
            f = lambda t: t.double()  # noqa: E731
            delta = f(Wm) - f(W_hat)
            out["requantize_gate"] = {
                "nf4_error_vs_weight": float((f(W_hat) - Wd.double()).norm() / Wd.double().norm()),
                "requant_error_vs_merged": float((f(back) - f(Wm)).norm() / f(Wm).norm()),
                "adapter_delta_norm_vs_weight": float(delta.norm() / f(Wm).norm()),
                "requant_error_vs_adapter_delta": float((f(back) - f(Wm)).norm() / delta.norm()),
                "codes_changed_fraction": float((qt2.codes != qt.codes).double().mean()),
            }
            log(f"[bench] re-quantized merge: {out['requantize_gate']}")
            del W_hat, qt2, back, delta
        del Wd, qt, A, B, Wm
    return out


def format_gemv_bytes(fmt, N, K, M):
    """Bytes the comparison-format GEMV must move: codes, fp32 block
    constants and X in; Y (bf16) out."""
    code_bytes = N * K if fmt == "int8" else N * K // 2
    return code_bytes + 4 * (N * K // 64) + 2 * M * K + 2 * M * N


def run_formats(torch, q, args):
    """The comparison formats (NF4 with double quantization off, absmax INT4
    and INT8, one fp32 constant per 64-block) on the 4096 x 4096 q_proj weight
    of the GEMV workload: reconstruction error of each against the fp32
    weight (NF4 with double quantization beside them), and the dequant-GEMV
    kernel time at M = 1 and 16 over copies that do not fit the last-level
    cache."""
    from workloads import Inputs

    w = Inputs(2)
    N, K = w.shape(0)
    Wd = torch.from_numpy(w.weight(0)).cuda()
    W64 = Wd.double()
    out = {"weight": [N, K], "formats": {}}
    rel = lambda a: float((a.double() - W64).norm() / W64.norm())  # noqa: E731
    # NF4 with double quantization, the main format
    qt = q.Nf4Tensor.empty(N, K)
    q.qlora_nf4_quantize(Wd, qt, q.workspace(q.qlora_nf4_sizes(N, K, 0, 1)["quantize_ws_bytes"]))
    back = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    q.qlora_dequantize(qt, back)
    out["nf4_dq_rel_error"] = rel(back)
    del qt
    for fmt in ("nf4", "int4", "int8"):
        copies = []
        for _ in range(args.gemv_copies):
            t = q.QTensor.empty(N, K, fmt)
            q.qlora_quantize_format(Wd, t)
            copies.append(t)
        q.qlora_dequantize_format(copies[0], back)
        rec = {"rel_error": rel(back), "bits_per_weight": (8 if fmt == "int8" else 4) + 32 / 64}
        for M in (1, 16):
            X = dev_bf16(torch, w.X(0, M))
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            n = args.gemv_iters
            evs = timed_events(torch, n)
            for i in range(10):
                q.qlora_gemv_format(copies[i % len(copies)], X, Y)
            torch.cuda.synchronize()
            for i in range(n):
                q.qlora_time_next_launch(q.QLORA_KERNEL_FORMAT_GEMV, *evs[i])
                q.qlora_gemv_format(copies[i % len(copies)], X, Y)
            torch.cuda.synchronize()
            med = statistics.median(a.elapsed_time(b) for a, b in evs)
            nbytes = format_gemv_bytes(fmt, N, K, M)
            gbs = nbytes / (med * 1e-3) / 1e9
            rec[f"gemv_m{M}"] = {"kernel_us_median": round(med * 1e3, 3), "bytes": nbytes,
                                 "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        out["formats"][fmt] = rec
        log(f"[bench] format {fmt}: {rec}")
        del copies
    return out


def run_cpu_breadth():
    """Oracle timings beyond the main step (numpy quantize runs on one core):
    quantize params/s on the tiny and q_proj shapes and on a 1024-row slice of
    a 65B-layer 8192-wide weight; fp64 forward + backward of one linear of the
    tiny workload (M = 32) and of the 7B-block and 65B-layer q_proj shapes at
    M = 512, whose weight is the unquantized draw (only the rate is kept)."""
    import numpy as np
    from oracle import linalg, nf4
    from workloads import Inputs, bf16_bits_to_f32

    out = {"quantize_params_per_s": {}, "fwd_bwd_TFLOP/s": {}}
    rng = np.random.default_rng(3)
    for label, (N, K) in (("tiny 256x256", (256, 256)), ("q_proj 4096x4096", (4096, 4096)),
                          ("65B q_proj rows 1024x8192", (1024, 8192))):
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        t0 = time.perf_counter()
        nf4.quantize(W)
        dt = time.perf_counter() - t0
        out["quantize_params_per_s"][label] = round(N * K / dt, 1)
    f64 = linalg.bf16_to_f64
    for widx, M in ((1, 32), (4, 512), (5, 512)):
        w = Inputs(widx)
        name, N, K = w.w.layers[0]
        r, alpha = w.w.rank, w.w.alpha
        Wb = w.weight(0)
        wh = (Wb if w.w.weight_dtype == "f32" else bf16_bits_to_f32(Wb)).astype(np.float64)
        X, dY = f64(w.X(0, M)), f64(w.dY(0, M))
        A, B = f64(w.lora_A(0)), f64(w.lora_B(0))
        t0 = time.perf_counter()
        linalg.linear_fwd(X, wh, A, B, alpha, r)
        linalg.linear_bwd(X, dY, wh, A, B, alpha, r)
        dt = time.perf_counter() - t0
        out["fwd_bwd_TFLOP/s"][f"workload {widx} {name} {N}x{K} M={M}"] = round(linear_flops(M, N, K, r) / dt / 1e12, 6)
        log(f"[bench] cpu oracle breadth: workload {widx} {name} ({dt:.1f}s)")
    return out


def run_cpu_baseline():
    """The oracle as it stands, timed on the host over one whole step of the
    same workload: for each of the three linears, quantize + dequantize + fp64
    forward + fp64 backward at M = 4096."""
    import numpy as np
    from oracle import linalg, nf4
    from workloads import Inputs

    w = Inputs(3)
    M, r, alpha = w.w.tokens[0], w.w.rank, w.w.alpha
    f64 = linalg.bf16_to_f64
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((p.get("num_threads", 0) for p in threadpool_info()
                            if p.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    dt, flops = 0.0, 0
    for li, (name, N, K) in enumerate(w.w.layers):
        W = w.weight(li)
        X, dY = f64(w.X(li, M)), f64(w.dY(li, M))
        A, B = f64(w.lora_A(li)), f64(w.lora_B(li))
        t0 = time.perf_counter()
        ref = nf4.quantize(W)
        wh = f64(nf4.dequantize(ref["codes"], ref["absmax_e4m3"], ref["dq_scale"],
                                ref["dq_mean"])).reshape(N, K)
        Y, T = linalg.linear_fwd(X, wh, A, B, alpha, r)
        dX, dA, dB = linalg.linear_bwd(X, dY, wh, A, B, alpha, r)
        dt += time.perf_counter() - t0
        assert np.isfinite(Y).all() and np.isfinite(dX).all()
        flops += linear_flops(M, N, K, r)
        log(f"[bench] cpu oracle: {name} done ({dt:.1f}s so far)")
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads or cores,
            "host_cores": cores, "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"one whole step of the same workload (gate, up, down; M={M}, r={r}): "
                      "numpy NF4+DQ quantize and dequantize (single-threaded numpy) + fp64 "
                      "forward and backward (BLAS on the listed threads); input generation "
                      "not timed"}


def copy_calibration(torch, q, mib):
    """The library's streaming copy of known size, three times, for scaling
    the HBM byte counters of a profiled run (each reads and writes `mib`
    MiB)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        q.qlora_bench_copy(src, dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {mib} MiB")
    del src, dst


def measured_peaks(torch, q):
    """In-run reference points beside the spec peaks: the library's
    register-only MFMA loop on every SIMD and its streaming copy of 1 GiB;
    torch's bf16 matmul (hipBLASLt) on the 7B MLP's largest product as
    context."""
    def med_ms(fn, n=10):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)

    sink = torch.zeros(2056, dtype=torch.float32, device="cuda")
    flop = {}

    def mfma():
        flop["n"] = q.qlora_bench_mfma_peak(20000, sink)

    mfma_ms = med_ms(mfma)
    # shader clock of the last loop: counter ticks / real-time seconds
    clk = sink[2048:].view(torch.int64).cpu().tolist()
    mfma_ghz = (clk[1] - clk[0]) / ((clk[3] - clk[2]) / (q.qlora_bench_wall_clock_khz() * 1e3)) / 1e9
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = med_ms(lambda: q.qlora_bench_copy(src, dst))
    del src, dst
    M, N, K = 4096, 11008, 4096
    a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    b = torch.randn(K, N, device="cuda").to(torch.bfloat16)
    mm_ms = med_ms(lambda: torch.matmul(a, b))
    del a, b
    out = {"mfma_loop_TFLOP/s": round(flop["n"] / (mfma_ms * 1e-3) / 1e12, 1),
           "mfma_loop_shader_clock_GHz": round(mfma_ghz, 3),
           # the dense bf16 rate at 2.5 PFLOP/s per 2.4 GHz, scaled to that clock
           "spec_peak_at_that_clock_TFLOP/s": round(PEAK_BF16_TFLOPS * mfma_ghz / 2.4, 1),
           "copy_GB/s": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
           "context_torch_bf16_matmul_TFLOP/s": round(2 * M * N * K / (mm_ms * 1e-3) / 1e12, 1),
           "context_torch_bf16_matmul_shape": [M, N, K]}
    log(f"[bench] measured peaks: {out}")
    return out


def run_bulk(torch, q, args):
    """NF4 + double quantization of streamed bf16 weights: each tensor of the
    list is drawn on the GPU (not timed), then quantized (timed with events
    attached to the quantize kernel).  The whole 6.7B and 65B lists; with
    --bulk-sample only the first block / layer of each plus the two padding
    matrices."""
    from workloads import bulk_tensors, device_normal

    out = {}
    for widx, label in ((4, "6.7B (7B block list)"), (5, "65B (65B layer list)")):
        tl = bulk_tensors(widx)
        if args.bulk_sample:
            tl = tl[:7] + tl[-2:]
        total_params, total_ms, nbytes = 0, 0.0, 0
        outs = {}
        for i, (name, N, K) in enumerate(tl):
            Wd = device_normal(torch, (N, K), 5000 + 7 * widx + (i % 9), 0.02)
            if (N, K) not in outs:
                outs[(N, K)] = (q.Nf4Tensor.empty(N, K), q.workspace(q.qlora_nf4_sizes(N, K, 0, 1)["quantize_ws_bytes"]))
            qt, ws = outs[(N, K)]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            b.record()
            q.qlora_time_next_launch(q.QLORA_KERNEL_QUANTIZE, a, b)
            q.qlora_nf4_quantize(Wd, qt, ws)
            torch.cuda.synchronize()
            # the quantize call is one main kernel plus the small double
            # quantization encode; the event pair brackets the main kernel
            total_ms += a.elapsed_time(b)
            total_params += N * K
            nbytes += int(N * K * (2 + 0.5 + 1 / 64)) + 4 * ((N * K // 64 + 255) // 256) + 4
            del Wd
        gbs = nbytes / (total_ms * 1e-3) / 1e9
        out[f"workload{widx}"] = {"list": label, "tensors": len(tl), "params": total_params,
                                  "quantize_kernel_ms": round(total_ms, 3), "bytes": nbytes,
                                  "params_per_s": round(total_params / (total_ms * 1e-3), 1),
                                  "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                                  "sample": "first block/layer + 2 padding matrices" if args.bulk_sample else "whole list"}
        log(f"[bench] bulk quantize workload {widx}: {total_params / 1e9:.2f}e9 params in {total_ms:.1f} ms, "
            f"{gbs:.0f} GB/s")
        del outs
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-adamw", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--no-formats", action="store_true")
    ap.add_argument("--no-f16", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-bulk", action="store_true")
    ap.add_argument("--bulk-sample", action="store_true", help="quantize one block / layer of the bulk lists only")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup (clock ramp-up)")
    ap.add_argument("--gemv-copies", type=int, default=64)
    ap.add_argument("--gemv-iters", type=int, default=200)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run three plain copies of MIB MiB first and three last (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_fine_tuning_amd as q

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, q, args.copy_calibration)
    mlp = run_step(torch, q, args)
    workloads = None if args.no_workloads else run_workloads(torch, q, args)
    sweep = None if args.no_sweep else run_m_sweep(torch, q, args)
    gemv = None if args.no_gemv else run_gemv(torch, q, args)
    bulk = None if args.no_bulk else run_bulk(torch, q, args)
    adamw = None if args.no_adamw else run_adamw(torch, q, args)
    merge = None if args.no_merge else run_merge(torch, q, args)
    formats = None if args.no_formats else run_formats(torch, q, args)
    f16_step = None
    if not args.no_f16:
        m16 = run_step(torch, q, args, f16=True, steps=5, warmup=2, with_quantize=False)
        f16_step = {"ms_per_step": round(m16["ms_per_step"], 4),
                    "TFLOP/s": round(m16["flops"] / (m16["ms_per_step"] * 1e-3) / 1e12, 2),
                    "fwd_gemm_ms": round(m16["per_kernel"]["fwd_gemm"]["avg_ms"], 4),
                    "dx_gemm_ms": round(m16["per_kernel"]["dx_gemm"]["avg_ms"], 4)}
        log(f"[bench] fp16 compute step: {f16_step}")
    # last: the register-only MFMA loop runs the chip at its power limit,
    # and the clocks take a while to recover after it
    peaks = measured_peaks(torch, q)
    for res in [mlp["roofline"]] + [v["roofline"] for v in (workloads or {}).values()]:
        res["frac_of_measured_mfma"] = round(res["achieved"] / peaks["mfma_loop_TFLOP/s"], 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline()
        cpu["breadth"] = run_cpu_breadth()
    if args.copy_calibration:
        copy_calibration(torch, q, args.copy_calibration)
    value = mlp["flops"] / (mlp["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mlp["ms_per_step"], 4),
        "step_ms": mlp["step_ms"],
        "settle_s": args.settle,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": "llama-7b MLP linears (gate, up 4096->11008; down 11008->4096), "
                               "step = fwd + bwd per linear of NF4+DQ weights quantized once",
                   "global_batch": 4, "seq_len": 1024, "tokens": mlp["M"], "lora_rank": mlp["r"],
                   "lora_alpha": mlp["alpha"], "layers": mlp["layers"],
                   "flop_per_step": mlp["flops"], "parallelism": "single GPU"},
        "roofline": mlp["roofline"],
        "step_with_quantize": {"ms": round(mlp["ms_per_step_with_quantize"], 4),
                               "TFLOP/s": round(mlp["flops"] / (mlp["ms_per_step_with_quantize"] * 1e-3) / 1e12, 2)},
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "gemv": gemv,
        "workloads": workloads,
        "m_sweep": sweep,
        "bulk_quantize": bulk,
        "adamw": adamw,
        "merge": merge,
        "formats": formats,
        "f16_step": f16_step,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in mlp["per_kernel"].items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
