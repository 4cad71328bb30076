"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only.  No fast-math and no FMA contraction, so every sum is
the plain left-to-right double sum the source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(out: str = LIB, mutate: int = 0, quiet: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-o", out + ".tmp", os.path.join(HERE, "oracle.c"), "-lm"]
    if mutate:
        cmd.insert(1, f"-DORC_MUTATE={int(mutate)}")
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(mutate=int(sys.argv[1]) if len(sys.argv) > 1 else 0)
