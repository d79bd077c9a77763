"""The header is a C interface: tests/c_abi/host_calls.c, a C99 program that
includes include/adam.h, builds with gcc under -std=c99 -pedantic -Werror
(the HIP runtime headers it pulls in are treated as system headers), links
against libadamw_mi355x.so with no C++ or Python in between, and makes the
calls that need no GPU.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "adamw_optimizer_step_tensor_amd")
LIB = os.path.join(PKG, "libadamw_mi355x.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c99_and_host_calls_work(tmp_path):
    assert os.path.exists(LIB), "library not built (run __graft_entry__.build())"
    exe = tmp_path / "host_calls"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-isystem", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "host_calls.c"), "-o", str(exe),
           f"-L{PKG}", "-l:libadamw_mi355x.so", f"-Wl,-rpath,{PKG}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, f"check {run.returncode} failed: {run.stdout}{run.stderr}"
    assert run.stdout.strip() == "ok"
