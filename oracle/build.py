"""Compiles the C oracle (test infrastructure only) into oracle/liboracle.so.

The flags are part of the oracle's definition: no fused multiply-add
(-ffp-contract=off) and no fast-math, so each float operation is one IEEE
binary32 operation rounded to nearest-even, in the printed order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "adam_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O2",
    "-std=c11",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fexcess-precision=standard",
    "-Wall",
    "-Wextra",
    "-Werror",
]


def build(verbose: bool = False, source: str = SOURCE, output: str = LIBRARY,
          werror: bool = True) -> str:
    """Compiles ``source`` (default: the oracle) into ``output``."""
    tmp = output + ".tmp"
    flags = CFLAGS if werror else [f for f in CFLAGS if f != "-Werror"]
    cmd = ["gcc", *flags, source, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
