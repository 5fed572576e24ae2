"""Builds libokls.so (HIP for gfx950) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/okls_api.cpp", "csrc/okls_kernels.hip"]
OUT = os.path.join(HERE, "libokls.so")


def hipcc_command(out=OUT):
    return ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *[os.path.join(HERE, s) for s in SOURCES], "-o", out]


def build(verbose=False):
    tmp = OUT + ".tmp"
    cmd = hipcc_command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
