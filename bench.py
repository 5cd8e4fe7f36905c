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
Also reported: the roofline of the dominant kernel (the gate_up GEMM,
timed with HIP events on the stream it runs on), per-linear kernel times,
and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8-dynamic linear TFLOP/s (prefill) + weight GB/s (decode), % of roofline"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def cpu_baseline(shapes, M, rows, col_frac):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="token rows of the CPU-oracle sample")
    ap.add_argument("--cpu-col-frac", type=float, default=0.25,
                    help="fraction of output channels in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); multi-GPU scaling is not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_dynamic_quantized_amd as F
    import synth
    from fp8_dynamic_quantized_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    F.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    shapes = synth.SHAPES["c2"]
    M = synth.M_OF["c2"][0]
    log(f"setup: {len(shapes)} linears, M={M}")
    layers = []
    for j, (name, K, N) in enumerate(shapes):
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

    def step(ev=None):
        for i, L in enumerate(layers):
            if ev is not None:
                ev[i][0].record()
            F.fp8_quant_act(L["x"], q=L["qx"], scale=L["sx"])
            if ev is not None:
                ev[i][1].record()
            F.fp8_gemm(L["qx"], L["sx"], L["qw"], L["sw"], y=L["y"])
            if ev is not None:
                ev[i][2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    quant_ms = np.zeros(len(layers))
    gemm_ms = np.zeros(len(layers))
    for k in range(args.steps):
        for i in range(len(layers)):
            quant_ms[i] += evs[k][i][0].elapsed_time(evs[k][i][1])
            gemm_ms[i] += evs[k][i][1].elapsed_time(evs[k][i][2])
    quant_ms /= args.steps
    gemm_ms /= args.steps

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
    value = flops_step * args.steps / dt / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B prefill linears, M=4096 tokens: qkv 4096->6144, "
                        "o 4096->4096, gate_up 4096->28672, down 14336->4096; "
                        "per-token dynamic / per-channel static E4M3, bf16 in/out",
            "M": M,
            "shapes": [[L["name"], L["K"], L["N"]] for L in layers],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_prefill_kernel<256,256> (gate_up 4096x4096->28672)",
            "achieved": round(achieved, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": None,
        },
        "per_linear": per_layer,
    }
    if not args.no_cpu_baseline:
        for L in layers:
            del L["x"], L["qw"], L["y"], L["qx"]
        torch.cuda.empty_cache()
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(shapes, M, args.cpu_rows, args.cpu_col_frac)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
