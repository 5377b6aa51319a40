"""Compile the fp64 CPU oracle (test infrastructure) into oracle/libssmref.so.

Plain gcc, no fast-math and no floating-point contraction, so every
operation rounds exactly as written in ssm_ref.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libssmref.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ssm_ref.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
