"""Builds libskgemm.so in-tree with hipcc for gfx950 (no GPU needed)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libskgemm.so")
# device-ceiling probes for the roofline (bench.py --ceiling), a library of their own
PROBE_LIB = os.path.join(HERE, "libskprobe.so")
PROBE_SOURCES = ["sk_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sk_kernels.hip", "sk_kernels_mx.hip", "sk_kernels_ksplit.hip", "sk_backward.hip", "sk_api.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep hipcc from emitting packed-fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared libraries; returns the GEMM library's path."""
    from concurrent.futures import ThreadPoolExecutor
    objs, cmds = [], []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        cmds.append(cmd)
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(cmds), 5)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    n = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:n]), (PROBE_LIB, objs[n:])):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
