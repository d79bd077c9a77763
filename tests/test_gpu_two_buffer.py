"""Two-buffer state on the GPU: each step reads one buffer set and writes the
other, and the state must sit in set (t & 1), bit for bit the oracle's
state after t steps, while the set the step read still holds the state
before it.  Covers fp32 state, 16-bit state and bf16 params with
remainders; aligned, peeled (one shared element offset per tensor) and
per-element (independent offsets per stream) layouts; the host step; the
capturable step with noop steps; and a HIP graph of one capturable step
replayed, whose side must follow the device counter."""
import zlib

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import HostTensor, host_tensors

pytestmark = pytest.mark.gpu

SIZES = [4096, 1000, 7, 0, 70001, 1 << 18, 513]
STORAGES = {
    "f32_bf16g_bf16out": dict(p_kind="f32", g_dtype="bf16", p_out="bf16"),
    "f32_f32g": dict(p_kind="f32", g_dtype="f32", p_out=False),
    "bf16_state_f16out": dict(p_kind="bf16", g_dtype="bf16", p_out="f16"),
    "f16_state_f32out": dict(p_kind="f16", g_dtype="f16", p_out="f32"),
    "remainders": dict(p_kind="bf16_rem", g_dtype="bf16", p_out=True),
}
STATE = ("p", "rem", "m", "v")


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


def layout(kind, n, rng):
    if kind == "aligned":
        return None
    roles = ("p", "rem", "m", "v", "g", "p_out")
    if kind == "peeled":
        return [{r: o for r in roles} for o in rng.integers(0, 70, n)]
    return [{r: int(rng.integers(0, 9)) for r in roles} for _ in range(n)]


def garbage(host):
    """The second set's starting contents: values no step would produce
    (reading them by mistake shows in every comparison)."""
    out = []
    for h in host:
        g = h.copy()
        for r in STATE:
            a = getattr(g, r)
            if a is not None and a.size:
                a.view(np.uint8)[...] = 0x7B
        out.append(g)
    return out


def read_set(dev, alt, side):
    """The state of set `side` (p, rem, m, v) with the param-out copy."""
    first = dev.readback()
    if side == 0:
        return first
    second = alt.readback()
    return [HostTensor(b.p, b.m, b.v, a.g, a.p_out, b.rem, None) for a, b in zip(first, second)]


def build(host, offsets, alt_host=None):
    dev = DeviceSet(host, offsets)
    alt = DeviceSet(alt_host if alt_host is not None else garbage(host), offsets)
    alts = [{r: d.get(r) for r in ("p", "m", "v", "rem")} for d in alt.tensors]
    for a, h in zip(alts, host):
        if h.p.size == 0:
            a.update(p=None, m=None, v=None, rem=None)
    tl = A.adam_tl_build(dev.tensors, desc_for(host), alternates=alts)
    return dev, alt, tl


@pytest.mark.parametrize("lay", ["aligned", "peeled", "per_element"])
@pytest.mark.parametrize("name", list(STORAGES))
def test_host_steps_alternate_between_the_sets(torch, name, lay):
    cfg = STORAGES[name]
    rng = np.random.default_rng(zlib.crc32(f"{name} {lay}".encode()))
    host = host_tensors(SIZES, seed=int(rng.integers(1 << 30)), m_v_init="random", **cfg)
    ref = copies(host)
    dev, alt, tl = build(host, layout(lay, len(SIZES), rng))
    assert tl.info()["two_buffer"] == 1
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, int(rng.integers(2)))
    orc = oracle.default()
    fn = A.adam_step_remainders if cfg["p_kind"] == "bf16_rem" else A.adam_step
    step, st = A.HostStep(0), [0]
    ot = oracle_tensors(ref)
    for t in range(1, 6):
        before = copies(ref)
        fn(tl, hl, 1.6e-3, step, 0.5)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5)
        torch.cuda.synchronize()
        assert step.value == st[0] == t
        assert_bitwise(read_set(dev, alt, t & 1), ref, ctx=f"{name} {lay} step {t}: the new state")
        assert_bitwise(read_set(dev, alt, (t - 1) & 1), before, roles=STATE,
                       ctx=f"{name} {lay} step {t}: the set read")
    tl.destroy()


@pytest.mark.parametrize("name", ["f32_bf16g_bf16out", "remainders", "bf16_state_f16out"])
def test_capturable_steps_and_graph_replays_follow_the_device_counter(torch, name):
    cfg = STORAGES[name]
    host = host_tensors(SIZES, seed=77, m_v_init="random", **cfg)
    ref = copies(host)
    dev, alt, tl = build(host, None)
    hl, hr = hp_pair(0.9, 0.999, 1e-8, 0.01, 1)
    orc = oracle.default()
    fn = A.adam_step_remainders_capturable if cfg["p_kind"] == "bf16_rem" else A.adam_step_capturable
    d_lr = torch.tensor([1e-3], dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_scale = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    ot, st = oracle_tensors(ref), [0]
    # eager capturable steps, the second a noop
    for noop in (0, 1, 0):
        d_noop.fill_(noop)
        fn(tl, hl, d_lr, d_step, d_scale, d_noop)
        orc.group_step(ot, hr, 1e-3, st, 2.0, noop=noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == st[0] == 2
    assert_bitwise(read_set(dev, alt, 0), ref, ctx=f"{name} eager")
    # one capturable step recorded, replayed with the flag and lr changed
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn(tl, hl, d_lr, d_step, d_scale, d_noop)
    torch.cuda.synchronize()
    for k, (noop, lr) in enumerate([(0, 1e-3), (0, 2e-3), (1, 2e-3), (0, 5e-4), (0, 5e-4)]):
        d_noop.fill_(noop)
        d_lr.fill_(lr)
        torch.cuda.synchronize()
        before = copies(ref)
        g.replay()
        torch.cuda.synchronize()
        orc.group_step(ot, hr, float(np.float32(lr)), st, 2.0, noop=noop)
        t = int(d_step.item())
        assert t == st[0]
        assert_bitwise(read_set(dev, alt, t & 1), ref, ctx=f"{name} replay {k}")
        if not noop:
            assert_bitwise(read_set(dev, alt, (t - 1) & 1), before, roles=STATE, ctx=f"{name} replay {k} read set")
    del g
    tl.destroy()


def test_sum_of_squares_and_scaled_state_with_two_buffers(torch):
    """The gradient reduction works on a two-buffer handle as on any other;
    scaled state cannot have two buffers."""
    host = host_tensors(SIZES, seed=5, g_dtype="bf16", p_kind="f32")
    dev, alt, tl = build(host, None)
    d = torch.zeros(1, dtype=torch.float64, device="cuda")
    A.adam_grad_sumsq(tl, d)
    torch.cuda.synchronize()
    want = sum(float(np.sum(((h.g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) ** 2))
               for h in host)
    assert abs(float(d.item()) - want) <= 1e-12 * want
    tl.destroy()
    sc = host_tensors([4096], seed=6, g_dtype="bf16", p_kind="f16_scaled", p_out="f16")
    dsc = DeviceSet(sc)
    alts = [dict(p=torch.zeros(4096, dtype=torch.float16, device="cuda"),
                 m=torch.zeros(4096, dtype=torch.float16, device="cuda"),
                 v=torch.zeros(4096, dtype=torch.float16, device="cuda"))]
    with pytest.raises(A.AdamError) as e:
        A.adam_tl_build(dsc.tensors, desc_for(sc), alternates=alts)
    assert e.value.status == A.ADAM_EINVAL
