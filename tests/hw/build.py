"""Builds tests/hw/libhw_accuracy.so (gfx950), the test-only library that
measures the hardware square root and reciprocal.

    python tests/hw/build.py   (__graft_entry__.build() runs it too)
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "hw_accuracy.hip")
LIBRARY = os.path.join(HERE, "libhw_accuracy.so")


def build(verbose: bool = False) -> str:
    import sys

    root = os.path.dirname(os.path.dirname(HERE))
    if root not in sys.path:
        sys.path.insert(0, root)
    from adamw_optimizer_step_tensor_amd import build as lib_build

    tmp = LIBRARY + ".tmp"
    cmd = [lib_build.hipcc(), f"--offload-arch={lib_build.ARCH}", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
