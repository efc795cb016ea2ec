"""Build the fp64 CPU oracle (`oracle/liboracle.so`) with the host C compiler.

Test infrastructure only: the product library never links or loads it.
No fast-math: the oracle must keep IEEE fp64 semantics.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
