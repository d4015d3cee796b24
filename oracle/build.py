"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``gn_oracle.c`` with gcc into ``libgn_oracle.so`` next to this file.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gn_oracle.c")
LIB = os.path.join(HERE, "libgn_oracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without -ffast-math: every fp64 operation stays as written
    # (no reassociation, no contraction into fused multiply-adds).
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
