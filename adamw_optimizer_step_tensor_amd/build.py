"""Builds libadamw_mi355x.so (HIP, gfx950) in-tree, next to this file.

    python -m adamw_optimizer_step_tensor_amd.build [-v] [-DADAM_UNROLL=4 ...]

Flags that define the arithmetic:
  -ffp-contract=off   every printed multiply and add is its own rounded
                      operation (no fused multiply-add);
  no fast-math        division and square root stay correctly rounded and
                      fp32 denormals are kept.
Packed fp32 instructions are disabled (-packed-fp32-ops).
The atomic optimizer is off: every atomic operation here is issued by one
lane, and the optimizer's rewrite uses its result at once, which would wait
for it where the one-pass kernel lets it complete under other work.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCE = os.path.join(PKG, "csrc", "adam.hip")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libadamw_mi355x.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False, extra=(), output: str = LIBRARY) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "-v"]
    build(verbose="-v" in sys.argv, extra=args)
