"""Build the plain-C oracle library (test infrastructure only).

gcc, strict IEEE fp32: no contraction of a*b+c into a fused multiply-add and
no fast-math, so every fp32 operation in the compressor is one rounding in the
order the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvarn_oracle.c")
LIB = os.path.join(HERE, "libkvarn_oracle.so")

FLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
    "-fno-unsafe-math-optimizations", "-Wall", "-Wextra", "-Wno-unused-parameter",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *FLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
