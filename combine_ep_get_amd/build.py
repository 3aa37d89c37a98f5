"""Build the gfx950 HIP library ``combine_ep_get_amd/_lib/libepget.so`` in-tree.

hipcc cross-compiles for gfx950 without a GPU.  ``-ffp-contract=off`` keeps
every float product and sum separately rounded (the combine contract);
packed-fp32 instruction selection is disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ep_get.hip")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libepget.so")
CEIL_SRC = os.path.join(HERE, "csrc", "ceiling.hip")
CEIL_LIB = os.path.join(LIBDIR, "libepceil.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, defines=(), out: str = LIB, src: str = SRC) -> str:
    """Compile ``src`` into ``out``; ``defines`` are extra -D flags."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIPFLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False):
    """The EP library and the HBM ceiling helper used by the benchmark."""
    return [build(verbose), build(verbose, out=CEIL_LIB, src=CEIL_SRC)]


if __name__ == "__main__":
    if len(sys.argv) > 1:
        print(build(verbose=True, defines=sys.argv[1:]))
    else:
        print(build_all(verbose=True))
