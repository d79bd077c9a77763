"""The update driven from C: tests/c_abi/gpu_step (built by
__graft_entry__.build() from tests/c_abi/gpu_step.c) is a C99 program that
uses only the HIP runtime and the C ABI -- no Python, no torch -- to copy
one fp32 tensor to the device, run several adam_step calls on a stream of
its own and copy the result back (also with the state in two buffer sets,
read back from set (step & 1)).  Its output must equal the oracle's, bit
for bit, and its host counter the number of steps."""
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import torch_mod
from workloads import host_tensors

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "gpu_step")


@pytest.mark.parametrize("mode,bias_correction,grad_scale,two", [(1, 1, 1.0, False), (0, 1, 0.5, False),
                                                                (1, 0, 2.0, False), (1, 1, 1.0, True)])
def test_c_client_matches_the_oracle(tmp_path, mode, bias_correction, grad_scale, two):
    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "tests/c_abi/gpu_step is not built (run __graft_entry__.build())"
    h = host_tensors([70001], g_dtype="f32", seed=95 + mode, m_v_init="random")[0]
    n, steps = h.p.size, 5
    lr, b1, b2, eps, wd = 1.6e-3, 0.9, 0.95, 1e-8, 0.1
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<q6f3i", n, lr, b1, b2, eps, wd, grad_scale, mode, bias_correction, steps))
        for a in (h.p, h.m, h.v, h.g):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    print(f"c client: n={n} steps={steps} mode={mode} bias_correction={bias_correction}", flush=True)
    run = subprocess.run([EXE, str(src), str(dst)] + (["two-buffer"] if two else []), capture_output=True,
                         text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    raw = np.fromfile(dst, np.uint8)
    got = raw[:3 * 4 * n].view(np.float32).reshape(3, n)
    got_step = int(raw[3 * 4 * n:].view(np.int32)[0])

    orc = oracle.default()
    ot = [oracle.OracleTensor(h.p.copy(), h.m.copy(), h.v.copy(), h.g, None, None, None)]
    st = [0]
    for _ in range(steps):
        orc.group_step(ot, oracle.HParams(b1, b2, eps, wd, mode, bias_correction), lr, st, grad_scale)
    assert got_step == st[0] == steps
    for row, want in zip(got, (ot[0].p, ot[0].m, ot[0].v)):
        assert np.array_equal(row.view(np.uint32), want.view(np.uint32))
