"""Compiles the input generator (``synth.c`` -> ``libsynth.so``) with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libsynth.so")
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", os.path.join(HERE, "synth.c"), "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
