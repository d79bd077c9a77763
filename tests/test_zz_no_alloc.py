"""adam_step_noalloc: adam_step without a handle, its work table in the
library's static device array (for callers that cannot allocate device
memory).  Its results must equal adam_step's on a handle of the same list,
bit for bit, call after call, also when a call's list is smaller than the
previous one's (the array keeps the previous table); lists beyond the
array's 65,536 records are refused before anything runs."""
import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import host_tensors

# fake, well-separated device addresses: these calls return before any
# memory is touched
BASE, STRIDE = 1 << 40, 1 << 32


def _fake(sizes):
    return [dict(p=BASE + (8 * i) * STRIDE, m=BASE + (8 * i + 1) * STRIDE, v=BASE + (8 * i + 2) * STRIDE,
                 g=BASE + (8 * i + 3) * STRIDE, numel=n) for i, n in enumerate(sizes)]


def _status(tensors, desc, step):
    try:
        A.adam_step_noalloc(tensors, desc, A.AdamHParams(), 1e-3, step, stream=0)
        return A.ADAM_OK
    except A.AdamError as e:
        return e.status


def test_noalloc_refuses_what_the_static_table_cannot_hold():
    step = A.HostStep(5)
    # 65,537 non-empty tensors need 65,537 records at any chunk
    assert _status(_fake([1] * 65537), A.make_desc(), step) == A.ADAM_ETOOBIG
    # a chunk the caller fixed is kept: 65,537 records of 1024 elements
    assert _status(_fake([1024 * 65537]), A.make_desc(chunk_elems=1024), step) == A.ADAM_ETOOBIG
    # storage schemes that adam_step does not take
    assert _status(_fake([8]), A.make_desc(p="bf16_rem"), step) == A.ADAM_EINVAL
    assert _status(_fake([8]), A.make_desc(p="f16_scaled"), step) == A.ADAM_EINVAL
    assert step.value == 5  # refused calls leave the counter
    assert "static scratch" in A.lib().adam_status_string(A.ADAM_ETOOBIG).decode()


def test_noalloc_empty_list_advances_the_counter():
    step = A.HostStep(0)
    for k in range(3):
        assert _status(_fake([0, 0]), A.make_desc(), step) == A.ADAM_OK
        assert step.value == k + 1
    step.value = 2 ** 31 - 1
    assert _status(_fake([0]), A.make_desc(), step) == A.ADAM_EINVAL


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


def _run(torch, host, hl, lr, steps, grad_scale, noalloc, **desc_kw):
    dev = DeviceSet(host)
    desc = desc_for(host, **desc_kw)
    step = A.HostStep(0)
    if noalloc:
        for _ in range(steps):
            A.adam_step_noalloc(dev.tensors, desc, hl, lr, step, grad_scale)
    else:
        tl = A.adam_tl_build(dev.tensors, desc)
        for _ in range(steps):
            A.adam_step(tl, hl, lr, step, grad_scale)
        torch.cuda.synchronize()
        tl.destroy()
    torch.cuda.synchronize()
    assert step.value == steps
    return dev.readback()


@pytest.mark.gpu
def test_noalloc_equals_adam_step_call_after_call(torch):
    """Two lists in a row through the static table, the second smaller (fewer
    tensors, fewer records), each for two steps: bit-identical to adam_step
    on a handle of the same list, and to the oracle."""
    orc = oracle.default()
    lists = [
        (host_tensors([70001, 4096 * 5, 123, 9, 65536 * 2, 4097, 1, 300000], g_dtype="bf16", p_out=True,
                      seed=61, m_v_init="random"), 1, dict()),
        (host_tensors([5000, 77, 4096], g_dtype="f32", seed=62, m_v_init="random"), 0, dict(chunk_elems=1024)),
        (host_tensors([20001, 3], g_dtype="f16", p_kind="bf16", p_out="f32", seed=63, m_v_init="random"), 1,
         dict()),
    ]
    for k, (host, mode, kw) in enumerate(lists):
        hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
        got = _run(torch, host, hl, 1.6e-3, 2, 0.5, True, **kw)
        want = _run(torch, host, hl, 1.6e-3, 2, 0.5, False, **kw)
        assert_bitwise(got, want, ctx=f"list {k}: noalloc vs adam_step")
        ref = copies(host)
        ot, st = oracle_tensors(ref), [0]
        for _ in range(2):
            orc.group_step(ot, hr, 1.6e-3, st, 0.5)
        assert_bitwise(got, ref, ctx=f"list {k}: noalloc vs oracle")


@pytest.mark.gpu
def test_noalloc_device_grad_scale_and_stream(torch):
    """A device grad scale and a stream of the caller's own; a step on a
    handle between two no-allocation calls does not disturb them."""
    host = host_tensors([9000, 513], g_dtype="bf16", p_out=True, seed=64, m_v_init="random")
    hl, _ = hp_pair(0.9, 0.999, 1e-8, 0.01, 1)
    s = torch.cuda.Stream()
    d_scale = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    a, b = DeviceSet(host), DeviceSet(host)
    desc = desc_for(host)
    tl = A.adam_tl_build(b.tensors, desc)
    sa, sb = A.HostStep(0), A.HostStep(0)
    for _ in range(3):
        A.adam_step_noalloc(a.tensors, desc, hl, 1e-3, sa, 7.0, d_scale, stream=s)
        A.adam_step(tl, hl, 1e-3, sb, 0.25, stream=s)
    s.synchronize()
    assert sa.value == sb.value == 3
    assert_bitwise(a.readback(), b.readback(), ctx="device grad scale, own stream")
    tl.destroy()
