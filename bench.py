#!/usr/bin/env python3
"""Benchmark: MoE-layer decode tokens/s and achieved HBM GB/s of the 4-bit
affine GEMV path on one MI355X.

Workload: one MoE layer decode step, batch 1 token -- hidden 2816, 128
experts, top-8 softmax routing with renormalisation, expert intermediate 704,
shared-expert intermediate 2112; 8-bit affine router, 4-bit affine (group
64) experts; bf16 activations ~N(0,1), fp32 accumulation; seeded synthetic
weights (the pages publish no dataset or checkpoint for this step).

One step = one token through the whole hot path of one layer (router GEMV,
softmax top-8, shared and 8 routed expert FFNs, weighted combine) in a single
launch of the library.  To measure HBM and not the 256 MB Infinity Cache,
the layer's weights are held in 32 separate copies (~14 GB) and consecutive
steps cycle through them, each with its own input token.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPIES = 32
N_TOKENS = 64


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(lw, X, seconds_hint: float = 15.0):
    """The fp64 oracle (as it stands) over a bounded sample of tokens of the
    same layer, threaded over tokens on the host cores."""
    import oracle

    L = oracle.OracleLayer(lw)
    cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    L.forward(X[0])
    one = time.perf_counter() - t0
    n = int(max(cores, min(4 * cores, seconds_hint * cores / max(one, 1e-3))))
    n = min(n, X.shape[0])
    threads = min(cores, n)
    t0 = time.perf_counter()
    oracle.forward_many(L, X[:n], threads=threads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode tokens of one layer (same shapes and weights), fp64 scalar C, "
                      f"{threads} threads over tokens"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phased", action="store_true",
                    help="time the three-launch variant instead of the single launch")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; multi-GPU runs are not "
                          "part of it (--gpus must be 1)"}))
        sys.exit(2)

    import torch

    import bit_quantized_gemv_amd as q
    import synth
    import synth.device as sd

    wl = synth.WORKLOADS["layer_decode"]
    log("generating layer weights")
    lw = synth.make_layer(wl, 0)
    algo_bytes = lw.algorithmic_bytes_decode()
    X = synth.make_tokens(wl, N_TOKENS, stream=1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"uploading {COPIES} copies of {lw.blobs.nbytes / 1e6:.0f} MB expert blobs")
    base = sd.DeviceLayer(lw)
    layers = [base]
    for i in range(1, COPIES):
        blobs = torch.empty_like(base.blobs)
        blobs.copy_(base.blobs)
        # router and shared expert are uploaded again per copy (own addresses)
        layers.append(sd.DeviceLayer(lw, blobs=blobs))
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    outs = torch.empty(N_TOKENS, wl.hidden, dtype=torch.int16, device=dev)
    idx = torch.empty(wl.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(wl.top_k, dtype=torch.float32, device=dev)
    ws = layers[0].layer.new_workspace(1)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i):
        L = layers[i % COPIES].layer
        t = i % N_TOKENS
        q.qmoe_moe_decode(L, Xd[t], None, False, outs[t], idx, w, ws, stream=sptr,
                          phased=args.phased)

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if q.qmoe_workspace_status(ws) != 0:
        raise SystemExit("device wait failure during warmup")

    # timed region: K steps; HIP events on the launch stream bracket each
    # step's launch(es) to time the kernel(s) themselves
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[2 * i].record(stream)
        step(args.warmup + i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code = q.qmoe_workspace_status(ws)
    if code != 0:
        raise SystemExit(f"device wait failure (code {code})")
    kern_ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(K)])
    kern_us = float(np.mean(kern_ms) * 1e3)
    kern_med_us = float(np.median(kern_ms) * 1e3)
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    tok_s = K / elapsed
    achieved = algo_bytes / (kern_us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.2f} us, kernel mean {kern_us:.2f} us median {kern_med_us:.2f} us, "
        f"{achieved:.0f} GB/s algorithmic")

    res = {
        "metric": "MoE-layer decode tokens/s + achieved HBM GB/s vs peak (4-bit affine GEMV)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 accumulation over u4/u8 affine codes, bf16 activations",
        "data": "synthetic (seeded; 4-bit/8-bit affine g64 weights, bf16 N(0,1) tokens)",
        "config": {"workload": "MoE layer decode, batch 1: hidden 2816, 128 experts, top-8, "
                               "expert inter 704, shared inter 2112, 8-bit router",
                   "launch": "phased (3 launches)" if args.phased else "single launch",
                   "weight_copies": COPIES, "algorithmic_bytes_per_step": algo_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "k_moe_step (whole decode step)",
                     "kernel_us_mean": kern_us, "kernel_us_median": kern_med_us},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(lw, X)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
