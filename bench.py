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
                on the stream it runs on; HBM traffic from the committed
                counter summary when it matches the current kernel source;
  per_linear    per-linear quantizer and GEMM kernel times;
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
  --summarize-profile DIR   per-kernel, per-grid duration / counter summary
                            of a rocprofv3 csv output directory.
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

    def step(ev=None):
        for i, L in enumerate(layers):
            if ev is not None:
                ev[i][0].record(stream)
            F.fp8_quant_act(L["x"], q=L["qx"], scale=L["sx"])
            if ev is not None:
                ev[i][1].record(stream)
            F.fp8_gemm(L["qx"], L["sx"], L["qw"], L["sw"], y=L["y"])
            if ev is not None:
                ev[i][2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for _ in layers] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    quant_ms = np.zeros(len(layers))
    gemm_ms = np.zeros(len(layers))
    for k in range(steps):
        for i in range(len(layers)):
            quant_ms[i] += evs[k][i][0].elapsed_time(evs[k][i][1])
            gemm_ms[i] += evs[k][i][1].elapsed_time(evs[k][i][2])
    quant_ms /= steps
    gemm_ms /= steps

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
    dom = [i for i, L in enumerate(layers) if L["name"] == "gate_up"][0]
    Ld = layers[dom]
    achieved = 2 * M * Ld["N"] * Ld["K"] / (gemm_ms[dom] * 1e-3) / 1e12
    res = {"M": M, "shapes": [[L["name"], L["K"], L["N"]] for L in layers],
           "value": flops_step * steps / dt / 1e12, "ms_per_step": dt / steps * 1e3,
           "achieved": achieved, "dom_us": gemm_ms[dom] * 1e3,
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


def summarize_profile(d):
    """Print per-kernel, per-grid-size averages of a rocprofv3 csv directory
    (kernel trace and/or counter collection)."""
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
                             * int(r["Grid_Size_Z"]),
                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if rows:
        agg = {}
        for name, grid, ns in rows:
            agg.setdefault((name, grid), []).append(ns)
        print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'grid':>10}  kernel")
        for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            print(f"{len(v):6d} {np.mean(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} "
                  f"{max(v) / 1e3:10.2f} {grid:10d}  {name[:110]}")
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        agg = {}
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"])
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
        print(f"{'calls':>6} {'avg':>14} {'grid':>10} {'counter':>12}  kernel")
        for (name, grid, cn), v in sorted(agg.items()):
            print(f"{len(v):6d} {np.mean(v):14.2f} {grid:10d} {cn:>12}  {name[:110]}")


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
    ap.add_argument("--summarize-profile", metavar="DIR")
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
