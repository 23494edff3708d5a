"""Builds liboracle.so (the CPU oracle) with gcc: scalar C, no FMA contraction,
no fast-math, OpenMP over the outer loops."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-fvisibility=hidden", os.path.join(HERE, "oracle.c"), "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
