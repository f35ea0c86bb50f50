"""Compile the CPU oracle (test infrastructure) into oracle/libnvfp4_oracle.so with gcc.

The oracle is plain C: no fast-math and no FMA contraction, so every fp32 step of the quantisation
recipe rounds on its own, as the recipe reads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")


def build(verbose: bool = False, extra_flags: tuple = (), out: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
