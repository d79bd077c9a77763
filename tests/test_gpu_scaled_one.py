"""One-pass scaled state: each workgroup updates a 4096-element tile once,
keeps the new p, m and v in registers, waits (a bounded wait) until the
last workgroup of its tensor has folded the tensor's maxima into scales,
and stores its tile; tiles whose wait runs out are recomputed and stored by
a follow-up pass.  Bit for bit against the oracle (values, scales and the
param-sync copy) and against the two-pass step, through host, capturable,
noop and graph-replayed steps; the follow-up pass is exercised by running
with no wait at all (every tile goes through it) and
with a 1 us wait."""
import time
import zlib

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import host_tensors

pytestmark = pytest.mark.gpu

# up to the one-pass limit of 2M elements per tensor, across tile, lane-group
# and record boundaries
SIZES = [0, 1, 3, 4, 5, 63, 64, 65, 511, 512, 513, 4095, 4096, 4097, 8191, 8193, 20001, 70001, 1 << 20,
         1 << 21]


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _host(p_kind, g_dtype, p_out, seed, sizes=SIZES):
    init = "large" if p_kind == "bf16_scaled" else "random"
    return host_tensors(sizes, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=seed, m_v_init=init,
                        g_std=1.0 if p_kind == "bf16_scaled" else 1e-3)


def _offsets(sizes, seed):
    """Every other tensor of 64 or more elements with all its buffers at one
    element offset 1..7 (a peeled head), the rest aligned: one pass takes
    lists whose tensors all allow 4-element accesses, which a tensor shorter
    than its head does not."""
    rng = np.random.default_rng(seed)
    roles = ("p", "m", "v", "g", "p_out")
    return [dict.fromkeys(roles, int(rng.integers(1, 8))) if i % 2 and n >= 64 else {}
            for i, n in enumerate(sizes)]


def _steps(torch, orc, host, hl, hr, steps, desc_kw, offsets=None, lr=1.6e-3, scale=0.5):
    ref = copies(host)
    dev = DeviceSet(host, offsets)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, **desc_kw))
    info = tl.info()
    step, st = A.HostStep(0), [0]
    ot = oracle_tensors(ref)
    for _ in range(steps):
        A.adam_step_scaled(tl, hl, lr, step, scale)
        orc.group_step(ot, hr, lr, st, scale)
    torch.cuda.synchronize()
    got = dev.readback()
    tl.destroy()
    return got, ref, info


@pytest.mark.parametrize("p_kind,g_dtype,p_out,mode", [
    ("f16_scaled", "bf16", "bf16", 1), ("f16_scaled", "f32", "f16", 0), ("bf16_scaled", "f16", "bf16", 1),
    ("bf16_scaled", "bf16", None, 0), ("f16_scaled", "f16", None, 1)])
@pytest.mark.parametrize("wait_us", [0, -1, 1])
def test_one_pass_matches_the_oracle(torch, orc, p_kind, g_dtype, p_out, mode, wait_us):
    host = _host(p_kind, g_dtype, p_out, zlib.crc32(f"{p_kind}{g_dtype}{p_out}{mode}".encode()) % 1000)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref, info = _steps(torch, orc, host, hl, hr, 3, dict(scaled_passes=1, scaled_wait_us=wait_us),
                            offsets=_offsets(SIZES, 5))
    assert (info["scaled_passes"], info["pieces"]) == (1, 1)
    assert_bitwise(got, ref, ctx=f"{p_kind}/{g_dtype}/{p_out}/{mode}/wait {wait_us}")


def test_one_pass_equals_two_passes(torch, orc):
    host = _host("f16_scaled", "bf16", "bf16", 91)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    one, ref, _ = _steps(torch, orc, host, hl, hr, 3, dict(scaled_passes=1))
    two, _, info = _steps(torch, orc, host, hl, hr, 3, dict(scaled_passes=2))
    assert info["scaled_passes"] == 2
    assert_bitwise(one, two, ctx="one pass vs two passes")
    assert_bitwise(one, ref, ctx="one pass vs oracle")


@pytest.mark.parametrize("grid,sizes,wait_us", [
    (1, [4096, 1, 4095, 77, 3000, 2], 0),               # one workgroup walks every tile
    (7, [4096 * 6, 5, 4096 * 3 + 1, 9000, 4096 * 6], 0),  # tensors of up to 7 tiles on 7 workgroups
    (7, [4096 * 6, 5, 4096 * 3 + 1, 9000, 4096 * 6], -1),
    (64, [1 << 17, 70001, 3, 1 << 17, 4097], 0)])
def test_one_pass_small_persistent_grids(torch, orc, grid, sizes, wait_us):
    """The persistent one-pass kernel on a grid capped at 1, 7 or 64
    workgroups (dispatch_tiles / 8), each workgroup taking many tiles in
    turn, a tensor's tiles spread over several rounds."""
    host = _host("f16_scaled", "bf16", "f16", 92, sizes=sizes)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref, info = _steps(torch, orc, host, hl, hr, 2,
                            dict(scaled_passes=1, dispatch_tiles=8 * grid, scaled_wait_us=wait_us))
    assert (info["scaled_passes"], info["dispatches"]) == (1, 1)
    assert_bitwise(got, ref, ctx=f"grid {grid}")


def test_one_pass_beside_another_kernel(torch, orc):
    """A one-pass step launched while matrix products on another stream hold
    the compute units, so that its persistent workgroups start over time
    rather than together: a wait for tiles of workgroups that have not
    started ends after a short grace and leaves its tile to the follow-up
    pass.  The results stay exact, and the step takes nowhere near its
    waits' full bound per tile."""
    sizes = [1 << 20] * 12 + [70001, 4097]
    host = _host("f16_scaled", "bf16", "bf16", 98, sizes=sizes)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, scaled_passes=1))
    assert tl.info()["scaled_passes"] == 1
    a = torch.randn(4096, 4096, device="cuda")
    side = torch.cuda.Stream()
    step, st = A.HostStep(0), [0]
    ot = oracle_tensors(ref)
    times = []
    for _ in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            prods = [a @ a for _ in range(4)]
        t0 = time.perf_counter()
        A.adam_step_scaled(tl, hl, 1.6e-3, step, 0.5)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        del prods
        orc.group_step(ot, hr, 1.6e-3, st, 0.5)
    got = dev.readback()
    tl.destroy()
    assert_bitwise(got, ref, ctx="beside matrix products")
    assert max(times) < 1.0, times


def test_one_pass_needs_tensors_within_two_rounds(torch):
    """A tensor whose tiles span 2 * grid positions or more: automatic mode
    takes two passes, and asking for one pass is refused."""
    host = _host("f16_scaled", "bf16", "f16", 96, sizes=[4096 * 20, 5])
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, dispatch_tiles=8 * 8))
    assert tl.info()["scaled_passes"] == 2
    tl.destroy()
    with pytest.raises(A.AdamError) as e:
        A.adam_tl_build(dev.tensors, desc_for(host, dispatch_tiles=8 * 8, scaled_passes=1))
    assert e.value.status == A.ADAM_EINVAL


def test_element_path_tensor_takes_two_passes(torch, orc):
    """A tensor whose buffers cannot share one aligned element takes the
    element path, which only the two-pass step has: the list runs in two
    passes, still exactly."""
    host = _host("f16_scaled", "bf16", "f16", 97, sizes=[70001, 4097, 300])
    offsets = [{}, {"p": 1, "m": 2, "v": 3, "g": 0, "p_out": 5}, {}]
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref, info = _steps(torch, orc, host, hl, hr, 2, dict(), offsets=offsets)
    assert info["scaled_passes"] == 2
    assert_bitwise(got, ref, ctx="element path")


@pytest.mark.parametrize("wait_us", [0, -1])
def test_one_pass_capturable_noop_and_graph_replay(torch, orc, wait_us):
    """Capturable one-pass steps (the second a noop: nothing written, the
    counts stay clear for the next step), then one capturable step recorded
    in a HIP graph and replayed three times with lr changed in between."""
    host = _host("f16_scaled", "bf16", "bf16", 93, sizes=[70001, 4096, 3, 1 << 20, 513])
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, scaled_passes=1, scaled_wait_us=wait_us))
    ot, st = oracle_tensors(ref), [0]
    d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_scale = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    for noop in (0, 1, 0, 0):
        d_noop.fill_(noop)
        A.adam_step_scaled_capturable(tl, hl, d_lr, d_step, d_scale, d_noop)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5, noop=noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == st[0] == 3
    assert_bitwise(dev.readback(), ref, ctx="capturable steps")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        A.adam_step_scaled_capturable(tl, hl, d_lr, d_step, d_scale, d_noop, stream=side)
    torch.cuda.synchronize()
    for lr in (1e-3, 2e-3, 5e-4):
        d_lr.fill_(lr)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        orc.group_step(ot, hr, float(np.float32(lr)), st, 0.5, noop=0)
        assert int(d_step.item()) == st[0]
        assert_bitwise(dev.readback(), ref, ctx=f"graph replay lr {lr}")
    del graph
    tl.destroy()


def test_one_pass_many_small_tensors_and_special_values(torch, orc):
    """300 tensors of 1..5000 elements (many tensors per dispatch group, most
    of one tile), with a NaN gradient in one tensor and an infinite one in
    another: those tensors' scales become NaN, the others are unaffected."""
    rng = np.random.default_rng(94)
    sizes = [int(x) for x in rng.integers(1, 5000, 300)]
    host = _host("f16_scaled", "f32", "f16", 95, sizes=sizes)
    host[10].g[0] = np.float32(np.nan)
    host[20].g[-1] = np.float32(np.inf)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref, info = _steps(torch, orc, host, hl, hr, 2, dict(scaled_passes=1))
    assert info["scaled_passes"] == 1
    assert np.isnan(ref[10].scales[0]) and np.isnan(ref[20].scales[1])
    assert_bitwise(got, ref, ctx="many small tensors")
