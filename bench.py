#!/usr/bin/env python3
"""Benchmark of the FP8-Dynamic linear on one MI355X.

A step is one pass of the hot path over the Llama-3.1-8B prefill linears at
M = 4096 tokens (qkv 4096->6144, o 4096->4096, gate_up 4096->28672,
down 14336->4096): for each, dynamic per-token E4M3 quantization of the bf16
activations followed by the FP8 MFMA GEMM with the fused per-token x
per-channel scale epilogue to bf16. Weights are quantized once, per output
channel, before timing (static weights). Inputs are seeded synthetic data
resident in HBM.

Prints one JSON line (value = whole-step TFLOP/s, 2*M*N*K per linear).
Also reported:
  roofline      the dominant kernel (the gate_up GEMM), timed with HIP events
                on the stream it runs on, around that launch only, in every
                timed step; HBM traffic from the committed counter summary
                when it matches the current kernel source;
  per_linear    per-linear quantizer and GEMM kernel times, from events around
                every launch in a separate pass after the timed steps (timed
                events in the stream leave short idle gaps between launches,
                which twelve of them per step would add to the step);
  decode        the Llama-3.1-70B decode linears at M in {1, 8, 32, 64}:
                end-to-end fp8_linear weight GB/s with cold weights
                (rotated copies well beyond the 256 MB last-level cache);
  block         the block variant on the Llama-3.2-3B linears at M = 8192:
                group-128 quantizer and block-scaled GEMM times, TFLOP/s;
  next_rows     SwiGLU->FP8 and RMSNorm->FP8 fused quantizers, percentile
                calibration over a 512 x 2048-token set, static quantization
                and the FP8 KV-cache write, in GB/s of algorithmic bytes;
  cpu_baseline  the CPU oracle timed on a bounded sample of the workload.

Other modes (profiling helpers, no JSON line):
  --copy-calibration        a plain 1 GiB device copy, three times, for
                            scaling the FETCH_SIZE / WRITE_SIZE counters;
  --profile-case CASE --profile-out DIR
                            one labelled workload for a rocprofv3 run (its
                            kernels and their algorithmic bytes per launch
                            go to DIR/case.json); CASE is one of
                              copy                  the 1 GiB copy, 3 times
                              decode:LINEAR:M       fp8_linear, 70B LINEAR at
                                                    M tokens, cold weights
                              quant:M:K             per-token quantizer, cold
                              prefill:LINEAR        8B prefill GEMM (codes in)
                              block:LINEAR          3B block GEMM (codes in);
  --summarize-profile DIR [DIR ...]
                            per-kernel, per-grid duration / counter summary
                            of rocprofv3 csv output directories; with
                            --profile-case directories, per case and kernel:
                            counter bytes (scaled by the copy case's) against
                            algorithmic bytes, clock and matrix-core busy
                            share, wave-state shares.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8-dynamic linear TFLOP/s (prefill) + weight GB/s (decode), % of roofline"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
DOM_KERNEL = "gemm_prefill_line_kernel<false, 256>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_prefill_line_gate_up_m4096_traffic.txt")
KERNEL_SOURCES = ["fp8_dynamic_quantized_amd/csrc/gemm_line.hpp",
                  "fp8_dynamic_quantized_amd/csrc/gemm_prefill.hip",
                  "fp8_dynamic_quantized_amd/csrc/device_common.hpp"]
COPY_BYTES = 1 << 30
PER_LINEAR_STEPS = 20       # steps of the per-linear pass (events around every launch)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is absent or was taken on other kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        if kv.get("kernel") != DOM_KERNEL:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(shapes, rows, col_frac):
    """The oracle (as it stands) on a bounded sample: `rows` tokens x
    N*col_frac output channels of each linear; weights quantized before
    timing, as on the GPU."""
    import oracle.fp8dq_oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    prepared = []
    flops = 0
    for j, (name, K, N) in enumerate(shapes):
        n = max(128, int(N * col_frac))
        d = synth.workload(2, j, M=rows)
        wb = d["w"][:n]
        qw, sw = O.quant_per_row(wb)
        prepared.append((d["x"], qw, sw))
        flops += 2 * rows * n * K
    t0 = time.perf_counter()
    for xb, qw, sw in prepared:
        qx, sx = O.quant_per_row(xb)
        O.linear_per_channel(qx, sx, qw, sw)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} tokens x {col_frac:.3f} of the output channels of each "
                      f"of the 4 linears (per-token quantization + exact GEMM + "
                      f"epilogue), {flops / 1e9:.1f} GFLOP in {dt:.2f} s; weight "
                      f"quantization before timing; host cores {os.cpu_count()}"}


def bench_prefill(F, torch, steps, warmup, only=None):
    import synth
    shapes = [s for s in synth.SHAPES["c2"] if only is None or s[0] in only]
    M = synth.M_OF["c2"][0]
    log(f"prefill setup: {len(shapes)} linears, M={M}")
    layers = []
    for name, K, N in shapes:
        j = [s[0] for s in synth.SHAPES["c2"]].index(name)
        d = synth.workload(2, j)
        x = to_dev(d["x"], torch)
        w = to_dev(d["w"], torch)
        qw, sw = F.fp8_quant_act(w)            # static per-channel weights
        del w
        layers.append({
            "name": name, "K": K, "N": N, "x": x, "qw": qw, "sw": sw,
            "qx": torch.empty((M, K), dtype=torch.uint8, device="cuda"),
            "sx": torch.empty((M,), dtype=torch.float32, device="cuda"),
            "y": torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
        })
    torch.cuda.synchronize()
    flops_step = sum(2 * M * L["N"] * L["K"] for L in layers)
    stream = torch.cuda.current_stream()        # the stream every launch uses

    dom = [i for i, L in enumerate(layers) if L["name"] == "gate_up"][0]

    def step(ev=None, every=False):
        # ev[i] = (before the quantizer, between, after the GEMM) of linear i;
        # recorded for the dominant linear's GEMM only, or (every) for all
        for i, L in enumerate(layers):
            if ev is not None and every:
                ev[i][0].record(stream)
            F.fp8_quant_act(L["x"], q=L["qx"], scale=L["sx"])
            if ev is not None and (every or i == dom):
                ev[i][1].record(stream)
            F.fp8_gemm(L["qx"], L["sx"], L["qw"], L["sw"], y=L["y"])
            if ev is not None and (every or i == dom):
                ev[i][2].record(stream)

    def new_events(n):
        return [[[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                 for _ in layers] for _ in range(n)]

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    evs = new_events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_ms = np.mean([evs[k][dom][1].elapsed_time(evs[k][dom][2]) for k in range(steps)])

    # per-linear breakdown: a separate pass, events around every launch
    diag = max(5, min(steps, PER_LINEAR_STEPS))
    evd = new_events(diag)
    for k in range(diag):
        step(evd[k], every=True)
    torch.cuda.synchronize()
    quant_ms = np.zeros(len(layers))
    gemm_ms = np.zeros(len(layers))
    for k in range(diag):
        for i in range(len(layers)):
            quant_ms[i] += evd[k][i][0].elapsed_time(evd[k][i][1])
            gemm_ms[i] += evd[k][i][1].elapsed_time(evd[k][i][2])
    quant_ms /= diag
    gemm_ms /= diag

    per_layer = {}
    for i, L in enumerate(layers):
        f = 2 * M * L["N"] * L["K"]
        qbytes = M * L["K"] * 3 + M * 4
        per_layer[L["name"]] = {
            "gemm_us": round(gemm_ms[i] * 1e3, 2),
            "gemm_tflops": round(f / (gemm_ms[i] * 1e-3) / 1e12, 1),
            "quant_us": round(quant_ms[i] * 1e3, 2),
            "quant_gbs": round(qbytes / (quant_ms[i] * 1e-3) / 1e9, 1),
        }
    Ld = layers[dom]
    achieved = 2 * M * Ld["N"] * Ld["K"] / (dom_ms * 1e-3) / 1e12
    res = {"M": M, "shapes": [[L["name"], L["K"], L["N"]] for L in layers],
           "value": flops_step * steps / dt / 1e12, "ms_per_step": dt / steps * 1e3,
           "achieved": achieved, "dom_us": dom_ms * 1e3,
           "dom_shape": (M, Ld["K"], Ld["N"]), "per_layer": per_layer}
    del layers
    torch.cuda.empty_cache()
    return res


def bench_decode(F, torch, batches=7, per_batch=20, warm=5):
    """fp8_linear on the 70B decode shapes, cold weights: enough distinct
    copies of the quantized weight rotate through to exceed 2 GB."""
    import synth
    stream = torch.cuda.current_stream()
    out = {}
    fracs = []
    for j, (name, K, N) in enumerate(synth.SHAPES["c3"]):
        log(f"decode setup: {name} {K}->{N}")
        w = to_dev(synth.workload(3, j, x=False)["w"], torch)
        qw, sw = F.fp8_quant_act(w)
        del w
        wbytes = N * K + 4 * N
        copies = max(2, -(-(2 << 30) // wbytes) + 1)
        qws = [qw] + [qw.clone() for _ in range(copies - 1)]
        for i, M in enumerate(synth.M_OF["c3"]):
            x = to_dev(synth.workload(3, j, i, w=False)["x"], torch)
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
            sx = torch.empty((M,), dtype=torch.float32, device="cuda")
            need = F.fp8_workspace_bytes(M, N, K)
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
            c = [0]

            def run():
                F.fp8_linear(x, qws[c[0] % copies], sw, y=y, qx_out=qx, sx_out=sx, ws=ws)
                c[0] += 1
            for _ in range(warm):
                run()
            times = []
            for _ in range(batches):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(per_batch):
                    run()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / per_batch)
            times.sort()
            us = statistics.median(times)
            gbs = wbytes / (us * 1e-6) / 1e9
            fracs.append(gbs / PEAK_HBM_GBS)
            out[f"{name}_M{M}"] = {
                "us": round(us, 2), "p10_us": round(times[0], 2),
                "p90_us": round(times[-1], 2), "weight_gbs": round(gbs, 1),
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
            log(f"  M={M}: {us:.1f} us, weight {gbs:.0f} GB/s")
            del x, y, qx, sx, ws
        del qws, qw, sw
        torch.cuda.empty_cache()
    out["mean_frac"] = round(float(np.mean(fracs)), 4)
    out["protocol"] = (f"fp8_linear end-to-end (quantize + GEMM [+ split-K reduce]); "
                       f"median of {batches} batches of {per_batch} launches after "
                       f"{warm} warm-ups; weight copies rotated, >2 GB per shape; "
                       f"weight bytes = N*K + 4*N")
    return out


def _time_us(torch, fn, reps=20, warm=3, batches=5):
    """Median over batches of the average duration of `reps` back-to-back
    launches (HIP events on the current stream)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    times = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    return statistics.median(times)


def bench_next_rows(F, torch):
    """The producers fused with the quantizer, static calibration and the
    FP8 KV-cache write, at Llama-3.1-8B sizes (HBM-bound: algorithmic bytes
    moved per launch / time)."""
    import synth
    out = {}

    def rec(name, us, nbytes, shape):
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "gbs": round(gbs, 1),
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": int(nbytes), "shape": shape}
        log(f"  {name}: {us:.1f} us, {gbs:.0f} GB/s")

    M, inner, hidden = 4096, 14336, 4096
    gu = to_dev(synth.activations(M, 2 * inner, 61, 62), torch)
    q = torch.empty((M, inner), dtype=torch.uint8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    us = _time_us(torch, lambda: F.fp8_silu_mul_quant(gu, q=q, scale=s))
    rec("silu_mul_quant", us, M * 2 * inner * 2 + M * inner + 4 * M,
        f"gate_up out [{M},{2 * inner}] -> codes [{M},{inner}]")
    del gu, q

    x = to_dev(synth.activations(M, hidden, 63, 64), torch)
    gamma = torch.ones(hidden, dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, hidden), dtype=torch.uint8, device="cuda")
    us = _time_us(torch, lambda: F.fp8_rmsnorm_quant(x, gamma, q=q, scale=s))
    rec("rmsnorm_quant", us, M * hidden * 3 + hidden * 2 + 4 * M,
        f"[{M},{hidden}] -> codes")

    # calibration set: 512 samples x 2048 tokens of one layer's input (4096 wide)
    ncal = 512 * 2048 * hidden
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed_of(6, 0, 0, 0))
    cal = (torch.randn((512 * 2048, hidden), generator=g, device="cuda")).to(torch.bfloat16)
    scale = torch.empty((1,), dtype=torch.float32, device="cuda")
    ws = torch.empty(F.fp8_calib_workspace_bytes(ncal), dtype=torch.uint8, device="cuda")
    us = _time_us(torch, lambda: F.fp8_calib_scale(cal, 1, 999, scale=scale, ws=ws), reps=3,
                  warm=1, batches=3)
    rec("calib_scale", us, 2 * ncal * 2, f"{ncal} values (512 x 2048 tokens x {hidden}), 2 passes")
    del cal, ws
    torch.cuda.empty_cache()
    us = _time_us(torch, lambda: F.fp8_quant_static(x, scale, q=q))
    rec("quant_static", us, M * hidden * 3, f"[{M},{hidden}] -> codes")
    del x, q

    T, width, n_slots = 4096, 8 * 128, 8192
    k = to_dev(synth.activations(T, width, 65, 66), torch)
    v = to_dev(synth.activations(T, width, 67, 68), torch)
    slots = torch.randperm(n_slots, generator=torch.Generator().manual_seed(69))[:T].cuda()
    kc = torch.empty((n_slots, width), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((n_slots,), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    us = _time_us(torch, lambda: F.fp8_kv_cache_quant(k, v, slots, kc, vc, ks, vs))
    rec("kv_cache_quant", us, 2 * (T * width * 3 + 4 * T) + 8 * T,
        f"K,V [{T},{width}] -> cache rows")
    del k, v, kc, vc
    torch.cuda.empty_cache()
    return out


def bench_block(F, torch):
    """Block variant on the Llama-3.2-3B shapes, M = 8192 tokens: group-128
    activation quantization and the block-scaled GEMM, each timed alone
    (median of batches of back-to-back launches, HIP events)."""
    import synth
    out = {}
    tot_flops = tot_us = 0.0
    M = synth.M_OF["c4"][0]
    for j, (name, K, N) in enumerate(synth.SHAPES["c4"]):
        log(f"block setup: {name} {K}->{N}, M={M}")
        d = synth.workload(4, j)
        x = to_dev(d["x"], torch)
        w = to_dev(d["w"], torch)
        qw, sw = F.fp8_quant_weight_block(w)
        del w
        qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sx = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        q_us = _time_us(torch, lambda: F.fp8_quant_act(x, group=128, q=qx, scale=sx))
        g_us = _time_us(torch, lambda: F.fp8_gemm_block(qx, sx, qw, sw, y=y))
        fl = 2 * M * N * K
        tot_flops += fl
        tot_us += q_us + g_us
        tf = fl / (g_us * 1e-6) / 1e12
        qbytes = 3 * M * K + 4 * M * (K // 128)
        out[name] = {"gemm_us": round(g_us, 2), "gemm_tflops": round(tf, 1),
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "quant_us": round(q_us, 2),
                     "quant_gbs": round(qbytes / (q_us * 1e-6) / 1e9, 1)}
        log(f"  {name}: GEMM {g_us:.1f} us ({tf:.0f} TFLOP/s), group quant {q_us:.1f} us")
        del x, qx, sx, y, qw, sw
        torch.cuda.empty_cache()
    out["linear_tflops"] = round(tot_flops / (tot_us * 1e-6) / 1e12, 1)
    out["protocol"] = ("fp8_quant_act(group 128) and fp8_gemm_block timed separately; "
                       "median of 5 batches of 20 launches; linear_tflops = all four "
                       "linears' flops over the sum of both times")
    return out


def bench_long_small(F, torch):
    """c5: the Llama-3.1-8B gate_up at M = 32768 tokens of Student-t(3)
    activations with zero rows and planted values past 448 (MFMA-bound);
    c1: one 4096 -> 1024 linear at M = 16 tokens (weight streaming, launch-
    latency-bound). Both are fp8_linear end to end (quantize + GEMM), also
    split into its two launches for c5. Medians of batches of back-to-back
    launches, HIP events."""
    import synth
    out = {}
    d = synth.workload(5, 0)
    M, K, N = d["M"], d["K"], d["N"]
    log(f"long-context setup: gate_up {K}->{N}, M={M} (Student-t, "
        f"{len(d['zero_rows'])} zero rows, {len(d['planted'])} planted values)")
    x = to_dev(d["x"], torch)
    w = to_dev(d["w"], torch)
    del d
    qw, sw = F.fp8_quant_act(w)
    del w
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    l_us = _time_us(torch, lambda: F.fp8_linear(x, qw, sw, y=y, qx_out=qx, sx_out=sx),
                    reps=5, warm=2, batches=5)
    q_us = _time_us(torch, lambda: F.fp8_quant_act(x, q=qx, scale=sx), reps=10, warm=2, batches=5)
    g_us = _time_us(torch, lambda: F.fp8_gemm(qx, sx, qw, sw, y=y), reps=5, warm=2, batches=5)
    fl = 2 * M * N * K
    out["c5_gate_up"] = {
        "linear_us": round(l_us, 1), "linear_tflops": round(fl / (l_us * 1e-6) / 1e12, 1),
        "frac": round(fl / (l_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "gemm_us": round(g_us, 1), "gemm_tflops": round(fl / (g_us * 1e-6) / 1e12, 1),
        "quant_us": round(q_us, 2), "quant_gbs": round((3 * M * K + 4 * M) / (q_us * 1e-6) / 1e9, 1),
        "shape": f"[{M},{K}] Student-t(3) x [{N},{K}] -> bf16 [{M},{N}]"}
    log(f"  c5 gate_up: linear {l_us:.0f} us ({fl / (l_us * 1e-6) / 1e12:.0f} TFLOP/s), "
        f"GEMM {g_us:.0f} us, quant {q_us:.1f} us")
    del x, qx, sx, y, qw, sw
    torch.cuda.empty_cache()

    d = synth.workload(1, 0)
    M, K, N = d["M"], d["K"], d["N"]
    log(f"small setup: {K}->{N}, M={M}")
    x = to_dev(d["x"], torch)
    # cold weights: rotate distinct quantized copies, >= 2 GB in all
    copies = max(2, (2 << 30) // (N * K) + 1)
    w = to_dev(d["w"], torch)
    qw0, sw = F.fp8_quant_act(w)
    del w
    qws = [qw0.clone() for _ in range(copies)]
    del qw0
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(16, F.fp8_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    it = [0]

    def run():
        F.fp8_linear(x, qws[it[0] % copies], sw, y=y, qx_out=qx, sx_out=sx, ws=ws)
        it[0] += 1
    us = _time_us(torch, run, reps=20, warm=5, batches=7)
    wbytes = N * K + 4 * N
    out["c1_single"] = {"linear_us": round(us, 2),
                        "weight_gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
                        "frac": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "shape": f"[{M},{K}] x [{N},{K}] -> bf16 [{M},{N}], "
                                 f"{copies} weight copies rotated"}
    log(f"  c1: linear {us:.1f} us, weight {wbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    del x, qws, y, qx, sx, ws
    torch.cuda.empty_cache()
    return out


def copy_calibration(torch):
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


PROFILE_REPS = {"copy": (0, 3), "decode": (4, 8), "quant": (4, 8), "prefill": (2, 4),
                "block": (2, 4), "groupquant": (4, 8), "next": (4, 8)}


def profile_case(case, out_dir, torch):
    """Run one labelled workload; write out_dir/case.json with the kernels it
    launches (name prefixes) and their algorithmic bytes and flops per launch."""
    import synth
    import fp8_dynamic_quantized_amd as F
    kind = case.split(":")[0]
    warm, reps = PROFILE_REPS[kind]
    kernels = []
    if kind == "copy":
        src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        run = lambda i: dst.copy_(src)                      # noqa: E731
        kernels.append({"match": "copyBuffer", "bytes": 2 * COPY_BYTES, "flops": 0,
                        "read": COPY_BYTES, "write": COPY_BYTES, "what": "1 GiB device copy"})
    elif kind == "decode":
        _, lin, ms = case.split(":")
        M = int(ms)
        j = [n for n, _, _ in synth.SHAPES["c3"]].index(lin)
        _, K, N = synth.SHAPES["c3"][j]
        w = to_dev(synth.workload(3, j, x=False)["w"], torch)
        qw, sw = F.fp8_quant_act(w)
        del w
        copies = max(2, -(-(2 << 30) // (N * K)) + 1)
        qws = [qw] + [qw.clone() for _ in range(copies - 1)]
        x = to_dev(synth.activations(M, K, 7 + M, 8 + K), torch)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sxv = torch.empty((M,), dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(16, F.fp8_workspace_bytes(M, N, K)), dtype=torch.uint8,
                         device="cuda")
        run = lambda i: F.fp8_linear(x, qws[i % copies], sw, y=y, qx_out=qx,   # noqa: E731
                                     sx_out=sxv, ws=ws)
        rd = N * K + 4 * N + M * K + 4 * M
        kernels.append({"match": "gemm_decode", "bytes": rd + 2 * M * N, "read": rd,
                        "write": 2 * M * N, "flops": 2 * M * N * K,
                        "what": f"70B {lin} {K}->{N} at M={M}: weights N*K + 4N, codes M*K + 4M, y 2MN"})
        kernels.append({"match": "quant_rows", "bytes": 3 * M * K + 4 * M, "read": 2 * M * K,
                        "write": M * K + 4 * M, "flops": 0,
                        "what": f"per-token quantizer {M}x{K}: x 2MK, codes MK, scales 4M"})
    elif kind == "quant":
        _, ms, ks = case.split(":")
        M, K = int(ms), int(ks)
        copies = max(2, -(-(1 << 30) // (2 * M * K)) + 1)
        xs = [to_dev(synth.activations(M, K, 9 + c, 10), torch) for c in range(min(copies, 3))]
        xs += [xs[c % 3].clone() for c in range(3, copies)]
        q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sc = torch.empty((M,), dtype=torch.float32, device="cuda")
        run = lambda i: F.fp8_quant_act(xs[i % copies], q=q, scale=sc)   # noqa: E731
        kernels.append({"match": "quant_rows", "bytes": 3 * M * K + 4 * M, "read": 2 * M * K,
                        "write": M * K + 4 * M, "flops": 0,
                        "what": f"per-token quantizer {M}x{K} read cold: x 2MK, codes MK, scales 4M"})
    elif kind == "groupquant":
        # the block variant's activation quantizer (128-wide groups) on the
        # Llama-3.2-3B inputs, rotated over > 1 GB so it reads from HBM
        _, ms, ks = case.split(":")
        M, K = int(ms), int(ks)
        copies = max(2, -(-(1 << 30) // (2 * M * K)) + 1)
        xs = [to_dev(synth.activations(M, K, 11 + c, 12), torch) for c in range(min(copies, 3))]
        xs += [xs[c % 3].clone() for c in range(3, copies)]
        q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sc = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
        run = lambda i: F.fp8_quant_act(xs[i % copies], group=128, q=q, scale=sc)   # noqa: E731
        kernels.append({"match": "quant_groups", "bytes": 3 * M * K + 4 * M * K // 128,
                        "read": 2 * M * K, "write": M * K + 4 * M * K // 128, "flops": 0,
                        "what": f"group-128 quantizer {M}x{K} read cold: x 2MK, codes MK, "
                                f"scales 4MK/128"})
    elif kind == "next":
        # the fused producers, static quantization, calibration and KV-cache
        # write at the sizes bench.py times (inputs resident, as there)
        _, row = case.split(":")
        M, inner, hidden = 4096, 14336, 4096
        if row == "silu":
            gu = to_dev(synth.activations(M, 2 * inner, 61, 62), torch)
            q = torch.empty((M, inner), dtype=torch.uint8, device="cuda")
            s = torch.empty((M,), dtype=torch.float32, device="cuda")
            run = lambda i: F.fp8_silu_mul_quant(gu, q=q, scale=s)   # noqa: E731
            rd, wr = M * 2 * inner * 2, M * inner + 4 * M
            match, what = "silu_mul_kernel", f"SwiGLU -> FP8: gate_up out [{M},{2 * inner}] bf16 in, codes [{M},{inner}] + scales out"
        elif row == "rms":
            x = to_dev(synth.activations(M, hidden, 63, 64), torch)
            gamma = torch.ones(hidden, dtype=torch.bfloat16, device="cuda")
            q = torch.empty((M, hidden), dtype=torch.uint8, device="cuda")
            s = torch.empty((M,), dtype=torch.float32, device="cuda")
            run = lambda i: F.fp8_rmsnorm_quant(x, gamma, q=q, scale=s)   # noqa: E731
            rd, wr = M * hidden * 2 + hidden * 2, M * hidden + 4 * M
            match, what = "rmsnorm_kernel", f"RMSNorm -> FP8: x [{M},{hidden}] + gamma in, codes + scales out"
        elif row == "static":
            x = to_dev(synth.activations(M, hidden, 63, 64), torch)
            s = torch.full((1,), 0.01, dtype=torch.float32, device="cuda")
            q = torch.empty((M, hidden), dtype=torch.uint8, device="cuda")
            run = lambda i: F.fp8_quant_static(x, s, q=q)   # noqa: E731
            rd, wr = M * hidden * 2 + 4, M * hidden
            match, what = "quant_static_kernel", f"static quantization [{M},{hidden}]: x in, codes out"
        elif row == "kv":
            T, width, n_slots = 4096, 8 * 128, 8192
            k = to_dev(synth.activations(T, width, 65, 66), torch)
            v = to_dev(synth.activations(T, width, 67, 68), torch)
            slots = torch.randperm(n_slots, generator=torch.Generator().manual_seed(69))[:T].cuda()
            kc = torch.empty((n_slots, width), dtype=torch.uint8, device="cuda")
            vc = torch.empty_like(kc)
            ks = torch.empty((n_slots,), dtype=torch.float32, device="cuda")
            vs = torch.empty_like(ks)
            run = lambda i: F.fp8_kv_cache_quant(k, v, slots, kc, vc, ks, vs)   # noqa: E731
            rd, wr = 2 * T * width * 2 + 8 * T, 2 * (T * width + 4 * T)
            match, what = "kv_quant_kernel", f"FP8 KV-cache write: K, V [{T},{width}] + slots in, cache rows + scales out"
        elif row == "calib":
            n = 64 * 2048 * hidden     # 2^29 values (the bench runs 8 times as many)
            g = torch.Generator(device="cuda")
            g.manual_seed(synth.seed_of(6, 0, 0, 0))
            cal = torch.randn((64 * 2048, hidden), generator=g, device="cuda").to(torch.bfloat16)
            s = torch.empty((1,), dtype=torch.float32, device="cuda")
            ws = torch.empty(F.fp8_calib_workspace_bytes(n), dtype=torch.uint8, device="cuda")
            run = lambda i: F.fp8_calib_scale(cal, 1, 999, scale=s, ws=ws)   # noqa: E731
            rd, wr = 2 * n, 0
            match, what = "calib_hist_kernel", (f"calibration histogram pass over {n} bf16 values "
                                                f"(two per call; the histograms are workspace)")
        else:
            raise SystemExit(f"unknown next-row case {row}")
        kernels.append({"match": match, "bytes": rd + wr, "read": rd, "write": wr, "flops": 0,
                        "what": what})
    elif kind in ("prefill", "block"):
        _, lin = case.split(":")
        c = 2 if kind == "prefill" else 4
        j = [n for n, _, _ in synth.SHAPES[f"c{c}"]].index(lin)
        _, K, N = synth.SHAPES[f"c{c}"][j]
        M = synth.M_OF[f"c{c}"][0]
        d = synth.workload(c, j)
        x, w = to_dev(d["x"], torch), to_dev(d["w"], torch)
        if kind == "prefill":
            qx, sxv = F.fp8_quant_act(x)
            qw, sw = F.fp8_quant_act(w)
            run = lambda i: F.fp8_gemm(qx, sxv, qw, sw)     # noqa: E731
            sbytes = 4 * (M + N)
            match = "gemm_prefill_line_kernel<false"
        else:
            qx, sxv = F.fp8_quant_act(x, group=128)
            qw, sw = F.fp8_quant_weight_block(w)
            run = lambda i: F.fp8_gemm_block(qx, sxv, qw, sw)   # noqa: E731
            sbytes = 4 * (M * K // 128 + (N // 128) * (K // 128))
            match = "gemm_prefill_line_kernel<true"
        del x, w
        rd = M * K + N * K + sbytes
        kernels.append({"match": match, "bytes": rd + 2 * M * N, "read": rd,
                        "write": 2 * M * N, "flops": 2 * M * N * K,
                        "what": f"{'8B' if c == 2 else '3B block'} {lin} M={M} {K}->{N}: "
                                f"codes MK + NK, scales, y 2MN"})
    else:
        raise SystemExit(f"unknown profile case {case}")
    for i in range(warm):
        run(i)
    torch.cuda.synchronize()
    for i in range(reps):
        run(warm + i)
    torch.cuda.synchronize()
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "case.json"), "w") as f:
        json.dump({"case": case, "warmup": warm, "launches": reps, "kernels": kernels}, f)
    log(f"profile case {case}: {warm} + {reps} launches")


def _read_profile_dir(d):
    """(case dict or None, {dispatch_id: (kernel, grid, ns)}, {dispatch_id: {counter: v}})"""
    case = None
    cj = os.path.join(d, "case.json")
    if os.path.exists(cj):
        with open(cj) as f:
            case = json.load(f)
    trace = {}
    for p in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                trace[int(r["Dispatch_Id"])] = (r["Kernel_Name"], grid,
                                                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    ctr = {}
    names = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                did = int(r["Dispatch_Id"])
                ctr.setdefault(did, {})[r["Counter_Name"]] = \
                    ctr.get(did, {}).get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                names[did] = (r["Kernel_Name"], int(r["Grid_Size"]))
    return case, trace, ctr, names


def summarize_profile(dirs):
    """Per-kernel, per-grid averages of rocprofv3 csv directories; for
    --profile-case directories, the per-case table of counter bytes against
    algorithmic bytes (and clock / matrix-core / wave-state shares)."""
    cases = {}
    for d in dirs:
        case, trace, ctr, names = _read_profile_dir(d)
        if case is None:
            # plain directory: per kernel and grid
            agg = {}
            for name, grid, ns in trace.values():
                agg.setdefault((name, grid), []).append(ns)
            print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'grid':>10}  kernel")
            for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
                print(f"{len(v):6d} {np.mean(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} "
                      f"{max(v) / 1e3:10.2f} {grid:10d}  {name[:110]}")
            # the prefill step of this benchmark launches, per step, the qkv
            # GEMM (256 x 192 tiles) and then o, gate_up and down (256 x 256
            # tiles, the same grid): the gate_up launches are the middle ones
            seq = [trace[k] for k in sorted(trace)]
            n_qkv = sum(1 for nm, _, _ in seq if "gemm_prefill_line_kernel<false, 192>" in nm)
            wide = [ns for nm, _, ns in seq if DOM_KERNEL in nm][: 3 * n_qkv]
            if n_qkv and len(wide) == 3 * n_qkv:
                gu = [ns / 1e3 for ns in wide[1::3]]
                print(f"# gate_up GEMM launches of the prefill steps ({len(gu)}, warm-up "
                      f"first): " + " ".join(f"{v:.1f}" for v in gu))
                for last in (20, 10):
                    if len(gu) >= last:
                        print(f"# gate_up GEMM, mean of the last {last} launches: "
                              f"{np.mean(gu[-last:]):.2f} us")
                # a default-protocol run ends with the per-linear pass of
                # PER_LINEAR_STEPS steps; the launches before it are the
                # warm-up and timed steps
                if len(gu) >= 2 * PER_LINEAR_STEPS:
                    timed = gu[-2 * PER_LINEAR_STEPS:-PER_LINEAR_STEPS]
                    print(f"# gate_up GEMM, mean of the {PER_LINEAR_STEPS} launches before the "
                          f"per-linear pass (the timed steps when --steps is "
                          f"{PER_LINEAR_STEPS}): {np.mean(timed):.2f} us")
                    print(f"# gate_up GEMM in the per-linear pass (events around every launch): "
                          f"mean {np.mean(gu[-PER_LINEAR_STEPS:]):.2f} us")
            cagg = {}
            for did, cv in ctr.items():
                for cn, v in cv.items():
                    cagg.setdefault((names[did][0], names[did][1], cn), []).append(v)
            if cagg:
                print(f"{'calls':>6} {'avg':>16} {'grid':>10} {'counter':>24}  kernel")
                for (name, grid, cn), v in sorted(cagg.items()):
                    print(f"{len(v):6d} {np.mean(v):16.2f} {grid:10d} {cn:>24}  {name[:110]}")
            continue
        ent = cases.setdefault(case["case"], {"case": case, "disp": {}})
        if not ctr:      # a kernel-trace run: the durations
            for did, (name, grid, ns) in trace.items():
                ent["disp"][("t", d, did)] = {"name": name, "grid": grid, "ns": ns, "ctr": {},
                                              "trace_run": True}
        for did, cv in ctr.items():
            ent["disp"][("c", d, did)] = {"name": names[did][0], "grid": names[did][1],
                                          "ns": trace[did][2] if did in trace else None,
                                          "ctr": dict(cv), "trace_run": False}
    if not cases:
        return
    # counter scaling from the copy case: known bytes / counter bytes
    scale = {"FETCH_SIZE": None, "WRITE_SIZE": None}
    if "copy" in cases:
        for cn in scale:
            v = [e["ctr"][cn] for e in cases["copy"]["disp"].values()
                 if cn in e["ctr"] and "copyBuffer" in e["name"]]
            if v:
                scale[cn] = COPY_BYTES / (float(np.mean(v)) * 1024.0)
        print(f"# counter scale factors (1 GiB copy: bytes / counter KiB x 1024): "
              f"FETCH_SIZE {scale['FETCH_SIZE']}, WRITE_SIZE {scale['WRITE_SIZE']}")
    for cname, ent in cases.items():
        if cname == "copy":
            continue
        case = ent["case"]
        print(f"\n## case {cname} ({case['launches']} timed launches after {case['warmup']})")
        for k in case["kernels"]:
            es = [e for e in ent["disp"].values() if k["match"] in e["name"]]
            if not es:
                print(f"  {k['match']}: no dispatches")
                continue
            # kernels launched once per run (set-up, e.g. the weight
            # quantization before a decode case) are left out
            per_run = case["warmup"] + case["launches"]
            runs = len({key[1] for key, e in ent["disp"].items()})
            names = sorted({e["name"] for e in es})
            for nm in names:
                ee = [e for e in es if e["name"] == nm]
                if len(ee) < per_run * max(1, runs) // 2:
                    continue
                tr = [e for e in ee if e["trace_run"]]
                dur = [e["ns"] / 1e3 for e in (tr or ee) if e["ns"] is not None]
                line = [f"  {nm[:100]}", f"    {k['what']}"]
                avg_us = float(np.median(dur)) if dur else None
                if avg_us:
                    line.append(f"    dispatches {len(ee)}, median duration {avg_us:.2f} us "
                                f"(min {min(dur):.2f}, max {max(dur):.2f})")
                alg = k["bytes"]
                line.append(f"    algorithmic: read {k['read'] / 1e6:.3f} MB, write "
                            f"{k['write'] / 1e6:.3f} MB, total {alg / 1e6:.3f} MB"
                            + (f", {k['flops'] / 1e9:.2f} GFLOP" if k["flops"] else ""))
                if avg_us:
                    line.append(f"    algorithmic rate {alg / avg_us / 1e3:.0f} GB/s "
                                f"({alg / avg_us / 1e3 / PEAK_HBM_GBS * 100:.1f} % of 8 TB/s)"
                                + (f", {k['flops'] / avg_us / 1e6:.0f} TFLOP/s "
                                   f"({k['flops'] / avg_us / 1e6 / PEAK_FP8_TFLOPS * 100:.1f} % of 5 PF)"
                                   if k["flops"] else ""))
                meas = {}
                for cn in ("FETCH_SIZE", "WRITE_SIZE"):
                    v = [e["ctr"][cn] for e in ee if cn in e["ctr"]]
                    if v and scale[cn]:
                        meas[cn] = float(np.mean(v)) * 1024.0 * scale[cn]
                if meas:
                    rd = meas.get("FETCH_SIZE")
                    wr = meas.get("WRITE_SIZE")
                    parts = []
                    if rd is not None:
                        parts.append(f"read {rd / 1e6:.3f} MB ({rd / k['read']:.2f}x)")
                    if wr is not None:
                        parts.append(f"write {wr / 1e6:.3f} MB ({wr / k['write']:.2f}x)" if k["write"]
                                     else f"write {wr / 1e6:.3f} MB (no algorithmic output)")
                    if rd is not None and wr is not None:
                        parts.append(f"total {(rd + wr) / 1e6:.3f} MB ({(rd + wr) / alg:.2f}x)")
                        if avg_us:
                            parts.append(f"{(rd + wr) / avg_us / 1e3:.0f} GB/s measured")
                    line.append("    counters (scaled): " + ", ".join(parts))
                g = [e["ctr"] for e in ee if "GRBM_GUI_ACTIVE" in e["ctr"]]
                if g and avg_us:
                    ga = float(np.mean([c["GRBM_GUI_ACTIVE"] for c in g]))
                    clk = ga / 8.0 / (avg_us * 1e3)        # 8 XCDs, GHz
                    line.append(f"    clock {clk:.2f} GHz (GRBM_GUI_ACTIVE / 8 XCDs / duration)")
                    mb = [c["SQ_VALU_MFMA_BUSY_CYCLES"] for c in g if "SQ_VALU_MFMA_BUSY_CYCLES" in c]
                    if mb:
                        per_simd = float(np.mean(mb)) / 1024.0
                        line.append(f"    matrix cores busy {per_simd / (ga / 8.0) * 100:.1f} % "
                                    f"(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / busy cycles)")
                w = [e["ctr"] for e in ee if "SQ_WAVE_CYCLES" in e["ctr"]]
                if w:
                    wc = float(np.mean([c["SQ_WAVE_CYCLES"] for c in w]))
                    shares = []
                    for cn, lab in (("SQ_WAIT_ANY", "waiting (s_waitcnt and other waits)"),
                                    ("SQ_WAIT_INST_ANY", "ready instruction not issued"),
                                    ("SQ_ACTIVE_INST_VALU", "issuing VALU"),
                                    ("SQ_ACTIVE_INST_LDS", "issuing LDS")):
                        v = [c[cn] for c in w if cn in c]
                        if v and wc > 0:
                            shares.append(f"{lab} {float(np.mean(v)) / wc * 100:.1f} %")
                    lds = [c["SQ_LDS_BANK_CONFLICT"] for c in w if "SQ_LDS_BANK_CONFLICT" in c]
                    if lds:
                        shares.append(f"SQ_LDS_BANK_CONFLICT {float(np.mean(lds)):.0f}")
                    line.append("    wave time (SQ_*/SQ_WAVE_CYCLES): " + ", ".join(shares))
                print("\n".join(line))
                if DOM_KERNEL in nm and "FETCH_SIZE" in meas and "WRITE_SIZE" in meas:
                    # the lines bench.py reads back for the roofline's traffic
                    print(f"kernel: {DOM_KERNEL}")
                    print(f"kernel_source_sha256: {kernel_source_hash()}")
                    print(f"fetch_bytes_per_launch: {meas['FETCH_SIZE']:.0f}")
                    print(f"write_bytes_per_launch: {meas['WRITE_SIZE']:.0f}")
                    print(f"traffic_bytes_per_launch: {meas['FETCH_SIZE'] + meas['WRITE_SIZE']:.0f}")


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="token rows of the CPU-oracle sample")
    ap.add_argument("--cpu-col-frac", type=float, default=0.625,
                    help="fraction of output channels in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-regime section")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the block-variant section (Llama-3.2-3B shapes)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the fused-producer / calibration / KV-cache section")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context (M = 32768) and 16-token sections")
    ap.add_argument("--linears", default="qkv,o,gate_up,down",
                    help="prefill linears to run (profiling runs that must tell "
                         "the gate_up launches apart: every per-channel linear "
                         "of this size launches the same grid); must include gate_up")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-profile", metavar="DIR", nargs="+")
    ap.add_argument("--profile-case", metavar="CASE")
    ap.add_argument("--profile-out", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the path is measured on one GPU only.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.profile_case:
        from fp8_dynamic_quantized_amd import build as B
        if not os.path.exists(B.LIB):
            B.build()
        profile_case(args.profile_case, args.profile_out or ".", torch)
        return

    import fp8_dynamic_quantized_amd as F
    import synth
    from fp8_dynamic_quantized_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    F.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    only = [s.strip() for s in args.linears.split(",") if s.strip()]
    if "gate_up" not in only:
        print("bench.py: --linears must include gate_up (the roofline kernel)", file=sys.stderr)
        sys.exit(2)
    pre = bench_prefill(F, torch, args.steps, args.warmup, only)
    M, K, N = pre["dom_shape"]
    out = {
        "metric": METRIC,
        "value": round(pre["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B prefill linears, M=4096 tokens: qkv 4096->6144, "
                        "o 4096->4096, gate_up 4096->28672, down 14336->4096; "
                        "per-token dynamic / per-channel static E4M3, bf16 in/out",
            "M": pre["M"],
            "shapes": pre["shapes"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": f"{DOM_KERNEL} (gate_up {M}x{K} -> {N})",
            "achieved": round(pre["achieved"], 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre["achieved"] / PEAK_FP8_TFLOPS, 4),
            "traffic": read_traffic(),
            "avg_launch_us": round(pre["dom_us"], 2),
        },
        "per_linear": pre["per_layer"],
        "per_linear_protocol": ("HIP events around every launch, in a pass after the timed "
                                "steps; the events leave short idle gaps between launches, so "
                                "the GEMMs there run at a higher clock than in the timed steps"),
    }
    if not args.no_decode:
        out["decode"] = bench_decode(F, torch)
    if not args.no_block:
        out["block"] = bench_block(F, torch)
    if not args.no_long:
        out["long_small"] = bench_long_small(F, torch)
    if not args.no_next:
        log("fused producers, calibration, KV cache ...")
        out["next_rows"] = bench_next_rows(F, torch)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(synth.SHAPES["c2"], args.cpu_rows,
                                           args.cpu_col_frac)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
