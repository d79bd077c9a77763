"""Builds tests/c_abi/gpu_step, the C99 client that runs the update on the
GPU through the C ABI (gcc; links the HIP runtime and libadamw_mi355x.so).

    python tests/c_abi/build.py   (__graft_entry__.build() runs it too)
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "gpu_step.c")
EXE = os.path.join(HERE, "gpu_step")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "adamw_optimizer_step_tensor_amd")
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-isystem", os.path.join(rocm, "include"), SOURCE, "-o", tmp,
           f"-L{pkg}", "-l:libadamw_mi355x.so", "-Wl,-rpath,$ORIGIN/../../adamw_optimizer_step_tensor_amd",
           f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
