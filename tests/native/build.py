"""Builds the test-only probe library tests/native/libmfma_numerics.so (gfx950).

    python tests/native/build.py
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmfma_numerics.so")


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", LIB + ".tmp", os.path.join(HERE, "mfma_numerics.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
