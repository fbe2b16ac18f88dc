"""Compile libqsa.so (all HIP kernels + the C ABI) for gfx950, in-tree.

hipcc cross-compiles without a GPU.  Packed-FP32 instructions are disabled
for all device code (-packed-fp32-ops); the host pass warns that it does not
know the feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqsa.so")
SOURCES = ["qsa_api.hip", "k_update.hip", "k_score.hip", "k_select.hip", "k_attend.hip", "k_chunk.hip",
           "k_decode.hip", "k_union.hip"]
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False, extra_flags=(), out=LIB):
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
