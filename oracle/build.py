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


# A second build of the same source with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only), loaded by the sanitizer test in
# a child process with the sanitizer runtimes preloaded.
SAN_LIB = os.path.join(HERE, "libkvarn_oracle_san.so")
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = ["gcc", *FLAGS, *(SAN_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
