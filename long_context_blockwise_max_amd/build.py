"""Build libpulsar.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Run as `python -m long_context_blockwise_max_amd.build`.  The library lands next
to this file; the Python binding loads it from there.
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpulsar.so")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed fp32 VALU forms stay disabled
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose=False, resource_usage=False):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + (["-Rpass-analysis=kernel-resource-usage"] if resource_usage else [])
    cmd += ["-I", os.path.join(HERE, "..", "include"), "-o", tmp] + srcs
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose or resource_usage:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv)
    print("built", LIB)
