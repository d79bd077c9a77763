"""The streaming-ceiling probe (tests/hw/stream_probe.hip) does what its
measurements claim: every element of every input stream is read and every
element of every output stream written, over full XCD run groups and the
tail of the grid."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "hw", "libstream_probe.so")
N = 512 * (8 * 64 * 3 + 5)  # three whole run groups of tiles and a tail of 5 tiles


@pytest.fixture(scope="module")
def env():
    from gpu_helpers import torch_mod

    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIBRARY):
        pytest.fail(f"{LIBRARY} is missing: build it with python tests/hw/build.py")
    lib = ctypes.CDLL(LIBRARY)
    lib.stream_probe_run.restype = ctypes.c_int
    lib.stream_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    return torch, lib


def _run(torch, lib, ins, outs, r, w, n, limit=0, sink=0):
    in_arr = (ctypes.c_void_p * max(len(ins), 1))(*[t.data_ptr() for t in ins])
    out_arr = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
    ms = ctypes.c_float(0.0)
    rc = lib.stream_probe_run(r, w, in_arr, out_arr, n, limit, 2, sink,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(ms))
    torch.cuda.synchronize()
    return rc, ms.value


@pytest.mark.parametrize("r,w,limit", [(4, 3, 7), (2, 2, 0), (0, 1, 0), (1, 1, 7)])
def test_probe_reads_and_writes_every_element(env, r, w, limit):
    torch, lib = env
    rng = np.random.default_rng(r * 10 + w)
    host = [rng.integers(-1000, 1000, N).astype(np.float32) for _ in range(r)]  # sums are exact
    ins = [torch.from_numpy(h).to("cuda") for h in host]
    outs = [torch.full((N,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(w)]
    rc, ms = _run(torch, lib, ins, outs, r, w, N, limit)
    assert rc == 0 and ms > 0
    total = np.zeros(N, np.float32)
    for h in host:
        total = total + h
    for k, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy(), total + np.float32(k))


def test_read_only_probe_reads_every_element(env):
    torch, lib = env
    host = np.arange(N, dtype=np.float32)
    ins = [torch.from_numpy(host).to("cuda")]
    out = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    rc, _ = _run(torch, lib, ins, [out], 1, 0, N, 7, sink=0)
    assert rc == 0 and bool((out == -1.0).all())  # nothing stored without the flag
    rc, _ = _run(torch, lib, ins, [out], 1, 0, N, 7, sink=1)
    assert rc == 0 and np.array_equal(out.cpu().numpy(), host)


def test_probe_rejects_bad_arguments(env):
    torch, lib = env
    t = torch.zeros(N, dtype=torch.float32, device="cuda")
    assert _run(torch, lib, [t], [t], 1, 1, N - 1)[0] == -1  # not whole tiles
    assert _run(torch, lib, [t], [t], 5, 1, N)[0] == -1  # too many streams
    assert _run(torch, lib, [], [t], 0, 0, N)[0] == -1  # nothing to do
    assert _run(torch, lib, [t[1:]], [t], 1, 1, N - 512)[0] == -1  # misaligned input
