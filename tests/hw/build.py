"""Builds the measurement-only libraries in tests/hw (gfx950):
libhw_accuracy.so, which measures the hardware square root and reciprocal,
and libstream_probe.so, the streaming-ceiling probes.

    python tests/hw/build.py   (__graft_entry__.build() runs it too)
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "hw_accuracy.hip")
LIBRARY = os.path.join(HERE, "libhw_accuracy.so")
PROBE_SOURCE = os.path.join(HERE, "stream_probe.hip")
PROBE_LIBRARY = os.path.join(HERE, "libstream_probe.so")


def build(verbose: bool = False) -> str:
    """Builds both libraries; returns the accuracy library's path."""
    _build_one(SOURCE, LIBRARY, "-O2", verbose)
    _build_one(PROBE_SOURCE, PROBE_LIBRARY, "-O3", verbose)
    return LIBRARY


def _build_one(source: str, library: str, opt: str, verbose: bool) -> str:
    import sys

    root = os.path.dirname(os.path.dirname(HERE))
    if root not in sys.path:
        sys.path.insert(0, root)
    from adamw_optimizer_step_tensor_amd import build as lib_build

    tmp = library + ".tmp"
    cmd = [lib_build.hipcc(), f"--offload-arch={lib_build.ARCH}", opt, "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", source, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, library)
    return library


if __name__ == "__main__":
    build(verbose=True)
