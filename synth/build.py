"""Builds the seeded input generator: libsynth_host.so (gcc) and libsynth_dev.so
(hipcc, gfx950).  Both compile synth_core.h, so their draws are bit-identical."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    host = os.path.join(HERE, "libsynth_host.so")
    dev = os.path.join(HERE, "libsynth_dev.so")
    _run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-fvisibility=hidden", os.path.join(HERE, "synth_host.c"), "-o", host + ".tmp"], verbose)
    os.replace(host + ".tmp", host)
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fvisibility=hidden", os.path.join(HERE, "synth_dev.hip"), "-o", dev + ".tmp"], verbose)
    os.replace(dev + ".tmp", dev)
    return host, dev


if __name__ == "__main__":
    print(build(verbose=True))
