"""Build libgrokmoe.so (the gfx950 HIP library behind include/grok_moe.h) and libgrokmoe_probe.so (the
measurement probes behind include/grok_moe_probe.h) in the package directory.

    python -m mixture_experts_transformer_gemv_amd.build      # or build() from Python

Every HIP source under csrc/ is compiled with hipcc for gfx950 into an object file, then linked into one
shared library; probe/ likewise into the probe library.  Packed-fp32 instructions are disabled for all device
code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
PROBE_SRC = os.path.join(PKG, "probe")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgrokmoe.so")
PROBE_LIB = os.path.join(PKG, "libgrokmoe_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def sources(directory: str = CSRC) -> list[str]:
    return sorted(os.path.join(directory, f) for f in os.listdir(directory) if f.endswith(".hip"))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP source and link libgrokmoe.so and libgrokmoe_probe.so; returns the layer library's path.
    Always rebuilds."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = FLAGS + list(extra_flags or [])

    def compile_one(src):
        sub = "probe_" if os.path.dirname(src) == PROBE_SRC else ""
        obj = os.path.join(BUILD_DIR, sub + os.path.basename(src)[:-4] + ".o")
        # the probes export only their C entry points (the trace probe compiles the layer's tile kernel source again)
        cmd = [cc, *flags, *(["-fvisibility=hidden"] if sub else []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    def link(objs, out):
        tmp = out + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {out} failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)

    srcs, psrcs = sources(CSRC), sources(PROBE_SRC)
    with ThreadPoolExecutor(min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(compile_one, srcs + psrcs))
    link(objs[:len(srcs)], LIB)
    link(objs[len(srcs):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
