"""Independent handles on independent streams: three tensor lists of
different storage (fp32 master with bf16 gradients and param-out, scaled
fp16 state, bf16 params with remainders stepped by the capturable call from
device scalars), each stepped on its own HIP stream with no synchronisation
between the streams, so their kernels overlap.  Each list must match its own
oracle run bit for bit; a handle's scratch (capture block, tile maxima) is
per handle, so concurrent handles do not interfere."""
import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import host_tensors

pytestmark = pytest.mark.gpu

SIZES = [1 << 20, 333333, 4097, 0, 70001]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


def test_three_handles_on_three_streams(torch):
    orc = oracle.default()
    hosts = {
        "plain": host_tensors(SIZES, g_dtype="bf16", p_out="bf16", seed=90, m_v_init="random"),
        "scaled": host_tensors(SIZES, g_dtype="bf16", p_kind="f16_scaled", p_out="f16", seed=91,
                               m_v_init="random"),
        "remainders": host_tensors(SIZES, g_dtype="bf16", p_kind="bf16_rem", p_out=True, seed=92),
    }
    refs = {k: copies(h) for k, h in hosts.items()}
    devs = {k: DeviceSet(h) for k, h in hosts.items()}
    tls = {k: A.adam_tl_build(devs[k].tensors, desc_for(hosts[k])) for k in hosts}
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_scale = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    steps = {"plain": A.HostStep(0), "scaled": A.HostStep(0)}
    torch.cuda.synchronize()
    streams = {k: torch.cuda.Stream() for k in hosts}
    n = 4
    for _ in range(n):
        A.adam_step(tls["plain"], hl, 1.6e-3, steps["plain"], 0.5, stream=streams["plain"])
        A.adam_step_scaled(tls["scaled"], hl, 1.6e-3, steps["scaled"], 0.5, stream=streams["scaled"])
        A.adam_step_remainders_capturable(tls["remainders"], hl, d_lr, d_step, d_scale,
                                          stream=streams["remainders"])
    torch.cuda.synchronize()
    assert steps["plain"].value == steps["scaled"].value == int(d_step.item()) == n
    for k in hosts:
        ot = oracle_tensors(refs[k])
        st = [0]
        for _ in range(n):
            if k == "remainders":
                orc.group_step(ot, hr, 1.6e-3, st, 0.5, noop=0)
            else:
                orc.group_step(ot, hr, 1.6e-3, st, 0.5)
        assert_bitwise(devs[k].readback(), refs[k], ctx=k)
        tls[k].destroy()


def test_four_host_threads_build_and_step_their_own_handles(torch):
    """Four host threads at once, each building its own handle and stepping
    it ten times on its own stream (fp32 master, capturable fp32 master,
    scaled bf16 state, bf16 params with remainders); the library keeps no
    state between handles, so each result matches its oracle run bit for
    bit."""
    import threading

    orc = oracle.default()
    kinds = {
        "plain": dict(p_kind="f32", p_out="f16", seed=93),
        "capturable": dict(p_kind="f32", p_out="bf16", seed=94),
        "scaled": dict(p_kind="bf16_scaled", p_out="bf16", seed=95),
        "remainders": dict(p_kind="bf16_rem", p_out=True, seed=96),
    }
    hosts = {k: host_tensors(SIZES, g_dtype="bf16", m_v_init="large" if k == "scaled" else "random",
                             g_std=1.0 if k == "scaled" else 1e-3, **kw)
             for k, kw in kinds.items()}
    refs = {k: copies(h) for k, h in hosts.items()}
    devs = {k: DeviceSet(h) for k, h in hosts.items()}
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    torch.cuda.synchronize()
    n = 10
    errors, counters = [], {}

    def work(k):
        try:
            stream = torch.cuda.Stream()
            tl = A.adam_tl_build(devs[k].tensors, desc_for(hosts[k]), stream=stream)
            if k == "capturable":
                d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
                d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
                stream.wait_stream(torch.cuda.current_stream())
                for _ in range(n):
                    A.adam_step_capturable(tl, hl, d_lr, d_step, stream=stream)
                stream.synchronize()
                counters[k] = int(d_step.item())
            else:
                fn = {"plain": A.adam_step, "scaled": A.adam_step_scaled,
                      "remainders": A.adam_step_remainders}[k]
                step = A.HostStep(0)
                for _ in range(n):
                    fn(tl, hl, 1.6e-3, step, stream=stream)
                stream.synchronize()
                counters[k] = step.value
            tl.destroy()
        except Exception as e:  # reported by the main thread
            errors.append((k, e))

    threads = [threading.Thread(target=work, args=(k,)) for k in kinds]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    assert counters == {k: n for k in kinds}
    for k in kinds:
        ot = oracle_tensors(refs[k])
        st = [0]
        for _ in range(n):
            orc.group_step(ot, hr, 1.6e-3, st, 1.0, noop=0 if k == "capturable" else None)
        assert_bitwise(devs[k].readback(), refs[k], ctx=k)
