"""Builds libw8a8moe.so, the gfx950 HIP library behind include/w8a8moe.h.

Flags: -ffp-contract=off and correctly rounded fp32 division keep every fp32
operation of the epilogues a single IEEE operation in the written order (the
quantization rule divides); packed fp32 instructions are disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "quant.hip", "route.hip", "align.hip", "gemm.hip"]
LIB = os.path.join(HERE, "libw8a8moe.so")
# measured-peak probes for the benchmark (include/w8a8probe.h), a library of their own
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libw8a8probe.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 8) -> str:
    _build(SOURCES, LIB, verbose, jobs)
    _build(PROBE_SOURCES, PROBE_LIB, verbose, jobs)
    return LIB


def _build(sources, lib, verbose: bool, jobs: int) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if out.strip():
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
