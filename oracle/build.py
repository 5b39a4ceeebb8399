"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only: nothing in the decode library builds against it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    # -ffp-contract=off: no fused multiply-add, every double op rounds as written
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-Wall", "-Wextra", "-fPIC",
           "-shared", "-pthread", "-o", tmp, os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
