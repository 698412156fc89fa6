"""Build libkvarn.so (the C ABI of include/kvarn.h) with hipcc for gfx950.

Each HIP source is compiled on its own and the objects are linked into one
shared library placed next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvarn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kvarn_api.hip", "compress.hip", "rotate.hip", "decode.hip", "decode_split.hip", "decode_wide.hip", "prefill.hip", "prefill_wide.hip", "window_mfma.hip"]
# measured floors for the benchmark (plain read, matrix-op rate, empty launch):
# a library of their own, not linked into libkvarn.so
FLOORS_SOURCE = "floors.hip"
FLOORS_LIB = os.path.join(HERE, "libkvarn_floors.so")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-op results in ordinary VGPRs: without it the compiler puts some
    # accumulators in AGPRs and copies every result out with one more vector
    # instruction (about 10% of the wide-head decode's per-tile instructions)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    f"-I{os.path.join(ROOT, 'include')}",
]
# The compressor must round every fp32 operation on its own (byte parity with
# the CPU oracle); the attention kernels may contract.
PER_FILE = {"compress.hip": ["-ffp-contract=off"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))] + [FLOORS_SOURCE]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], FLOORS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
