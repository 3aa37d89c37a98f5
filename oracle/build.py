"""Compile the C oracle (and its threaded driver) into ``oracle/liboracle.so``
(gcc, no FMA contraction).

TEST INFRASTRUCTURE: the oracle is only loaded by the tests, the smoke check and
the CPU-baseline leg of the benchmark.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
MT_SRC = os.path.join(HERE, "oracle_mt.c")   # threaded driver over the same functions
LIB = os.path.join(HERE, "liboracle.so")
LIBS = ["-lm", "-lpthread"]

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, MT_SRC, "-o", tmp, *LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
