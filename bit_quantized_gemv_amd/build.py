"""Build libqmoe.so (the gfx950 HIP library behind include/qmoe.h) in-tree.

    python -m bit_quantized_gemv_amd.build          # or build() from Python
    python -m bit_quantized_gemv_amd.build --trace  # libqmoe_trace.so: the same
        library with per-block phase timestamps in the decode step kernel
        (qmoe_trace_set); the binding loads it when QMOE_LIB names it
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqmoe.so")
TRACE_LIB = os.path.join(PKG, "libqmoe_trace.so")
SOURCES = ["qmoe_api.hip", "qmoe_decode.hip", "qmoe_router.hip", "qmoe_prefill.hip", "qmoe_pool.hip",
           "qmoe_sample.hip", "qmoe_attn.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # no packed fp32 math in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose: bool = False, trace: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    out = TRACE_LIB if trace else LIB
    extra = ["-DQMOE_TRACE"] if trace else []
    tag = ".trace" if trace else ""
    objs = []
    procs = []
    for s in srcs:
        o = os.path.join(CSRC, os.path.basename(s) + tag + ".o")
        cmd = [hipcc()] + flags() + extra + ["-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), s))
        objs.append(o)
    errs = []
    for p, s in procs:
        _, err = p.communicate()
        if p.returncode != 0:
            errs.append(f"{s}:\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
