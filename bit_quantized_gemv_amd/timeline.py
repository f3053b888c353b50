"""Per-block phase timeline of the one-launch decode step.

Runs the trace build of the library (``libqmoe_trace.so``, made by
``python -m bit_quantized_gemv_amd.build --trace``): every block of the step
kernel records s_memrealtime stamps (100 MHz, one clock for all CUs) at its
phase boundaries, kept in LDS while it works and written out when it ends.
This script runs the full-size layer (hidden 2816, 128 experts, top-8,
expert width 704, shared width 2112) over 32 weight copies cycled past the
MALL, 64 tokens, and prints per role the median, 95th percentile and maximum
of each stamp over blocks and launches, in µs from the first block's start.

    python -m bit_quantized_gemv_amd.timeline [--launches N]

Roles and stamps (see the step kernel's source for their exact places):
R router, S shared gate/up, G routed gate/up, D down + combine.
"""
from __future__ import annotations

import argparse
import ctypes as C
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRACE_LIB = os.path.join(ROOT, "bit_quantized_gemv_amd", "libqmoe_trace.so")

NAMES = {
    "R": {1: "weight loads issued", 4: "input staged", 2: "logits computed", 3: "logits published",
          9: "end"},
    "S": {1: "weight loads issued", 2: "input staged", 4: "computed", 5: "published", 9: "end"},
    "G": {2: "input staged", 10: "routing seen", 12: "top-k select", 13: "top-k gather",
          14: "top-k rank", 11: "top-k done", 3: "routing known", 1: "weight loads issued",
          4: "computed", 5: "published", 9: "end"},
    "D": {1: "shared weights issued", 10: "routing seen", 11: "top-k done", 2: "routing known",
          3: "shared flags seen", 4: "shared staged", 5: "routed flags seen", 6: "routed staged",
          7: "combined", 8: "output stored", 9: "end"},
}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--launches", type=int, default=64)
    ap.add_argument("--copies", type=int, default=32)
    args = ap.parse_args(argv)
    if not os.path.exists(TRACE_LIB):
        print(f"{TRACE_LIB} is missing: python -m bit_quantized_gemv_amd.build --trace",
              file=sys.stderr)
        return 2
    if os.environ.get("QMOE_LIB") != TRACE_LIB:
        # the package loads its library when imported (``-m`` imports it
        # first): run again in a child process that names the trace build
        import subprocess

        env = dict(os.environ, QMOE_LIB=TRACE_LIB)
        return subprocess.call([sys.executable, "-m", "bit_quantized_gemv_amd.timeline"] +
                               list(sys.argv[1:] if argv is None else argv), env=env, cwd=ROOT)
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bit_quantized_gemv_amd as q
    import synth
    import synth.device as sd

    wl = synth.WORKLOADS["layer_decode"]
    # blocks per role (8 router rows, 16 gate/up rows and 8 output rows a block)
    nR = -(-wl.n_experts // 8)
    perG = wl.inter // 16
    nS, nG, nD = wl.shared_inter // 16, wl.top_k * perG, wl.hidden // 8
    blocks = nR + nS + nG + nD
    slots = 256
    buf = torch.zeros(slots * blocks * 16, dtype=torch.int64, device="cuda")
    lib = q.lib()
    lib.qmoe_trace_set.argtypes = [C.c_void_p, C.c_int32]
    rc = lib.qmoe_trace_set(buf.data_ptr(), slots)
    if rc != 0:
        print(f"qmoe_trace_set: {q.STATUS_NAMES.get(rc, rc)}", file=sys.stderr)
        return 1
    lw = synth.make_layer(wl, 0)
    base = sd.DeviceLayer(lw)
    layers = [base]
    for _ in range(1, args.copies):
        b = torch.empty_like(base.blobs)
        b.copy_(base.blobs)
        layers.append(sd.DeviceLayer(lw, blobs=b))
    X = torch.from_numpy(synth.make_tokens(wl, 64, stream=1).view(np.int16)).cuda()
    out = torch.empty(wl.hidden, dtype=torch.int16, device="cuda")
    idx = torch.empty(wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.top_k, dtype=torch.float32, device="cuda")
    ws = base.layer.new_workspace(1)
    n_warm = max(args.copies, 64) * 2
    for i in range(n_warm):
        q.qmoe_moe_decode(layers[i % args.copies].layer, X[i % 64], None, False, out, idx, w, ws)
    torch.cuda.synchronize()
    g0 = q.qmoe_workspace_tag_counter(ws)
    N = min(args.launches, slots)
    for i in range(N):
        q.qmoe_moe_decode(layers[i % args.copies].layer, X[i % 64], None, False, out, idx, w, ws)
    torch.cuda.synchronize()
    assert q.qmoe_workspace_status(ws) == 0
    tr = buf.cpu().numpy().reshape(slots, blocks, 16)
    roles = {"R": range(0, nR), "S": range(nR, nR + nS), "G": range(nR + nS, nR + nS + nG),
             "D": range(nR + nS + nG, blocks)}
    vals, ends, starts, g_rank = {}, [], [], {}
    for k in range(N):
        t = tr[(g0 + k) % slots]  # call k matched its flags against tag g0 + k + 1
        t0 = t[:, 0][t[:, 0] > 0].min()
        ends.append((t[:, 9].max() - t0) / 100.0)
        starts.append((t[:, 0] - t0) / 100.0)
        for r, rng in roles.items():
            for i in NAMES[r]:
                v = t[list(rng), i]
                v = v[v > 0]
                if len(v):
                    vals.setdefault((r, i), []).append((v - t0) / 100.0)
        for j, b in enumerate(roles["G"]):
            g_rank.setdefault(j // perG, []).append((t[b, 5] - t0) / 100.0)
    st = np.concatenate(starts)
    print(f"decode step, {wl.hidden}x{wl.n_experts} experts top-{wl.top_k}, {N} launches "
          f"({args.copies} weight copies); blocks R {nR} S {nS} G {nG} D {nD}")
    print(f"last block end: median {np.median(ends):.2f} us, p10 {np.percentile(ends, 10):.2f}, "
          f"p90 {np.percentile(ends, 90):.2f}; block start: median {np.median(st):.2f}, "
          f"max {st.max():.2f}")
    print(f"{'role':4s} {'phase':24s} {'median':>7s} {'p95':>7s} {'max':>7s}  (us)")
    for r in roles:
        for i, nm in NAMES[r].items():
            if (r, i) not in vals:
                continue
            v = np.concatenate(vals[(r, i)])
            print(f"{r:4s} {nm:24s} {np.median(v):7.2f} {np.percentile(v, 95):7.2f} {v.max():7.2f}")
    print("G published, median by expert rank: " +
          " ".join(f"{r}:{np.median(v):.2f}" for r, v in sorted(g_rank.items())))
    return 0


if __name__ == "__main__":
    sys.exit(main())
