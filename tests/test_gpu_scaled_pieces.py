"""Two-pass scaled state on a list large enough (>= 4M elements in two or
more tensors) that the step runs in pieces of consecutive tensors pipelined
over two streams: the results must still equal the oracle's bit for bit (values,
scales and the param-sync copy), through the host step, the capturable step
with a noop step, and a HIP graph of one capturable step replayed."""
import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import host_tensors

pytestmark = pytest.mark.gpu

SIZES = [1 << 20, 700001, 1 << 20, 3, 900000, 1 << 20, 65536]  # 4.9M elements, 7 tensors


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


@pytest.mark.parametrize("p_kind,g_dtype,p_out", [("f16_scaled", "bf16", "f16"), ("bf16_scaled", "f32", "bf16")])
def test_pipelined_scaled_steps_match_the_oracle(torch, p_kind, g_dtype, p_out):
    init = "large" if p_kind == "bf16_scaled" else "random"
    host = host_tensors(SIZES, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=321, m_v_init=init,
                        g_std=1.0 if p_kind == "bf16_scaled" else 1e-3)
    assert sum(SIZES) >= 1 << 22
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, scaled_passes=2))
    assert tl.info()["scaled_passes"] == 2 and tl.info()["pieces"] > 1
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    orc = oracle.default()
    ot, st = oracle_tensors(ref), [0]
    # host steps
    step = A.HostStep(0)
    for _ in range(2):
        A.adam_step_scaled(tl, hl, 1.6e-3, step, 0.5)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5)
    torch.cuda.synchronize()
    assert_bitwise(dev.readback(), ref, ctx="host steps")
    # capturable steps, the second a noop
    d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
    d_step = torch.tensor([st[0]], dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_scale = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    for noop in (0, 1, 0):
        d_noop.fill_(noop)
        A.adam_step_scaled_capturable(tl, hl, d_lr, d_step, d_scale, d_noop)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5, noop=noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == st[0]
    assert_bitwise(dev.readback(), ref, ctx="capturable steps")
    # one capturable step recorded in a graph, replayed with lr changed
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


@pytest.mark.parametrize("sizes,pieces,dispatch_tiles,dispatches", [
    # two tensors, one of them a single element: one piece (the element
    # alone would be a piece of 32 tiles)
    ([(1 << 22) + 4097, 1], 1, 0, 1),
    ([1] * 9 + [(1 << 22) + 3], 1, 0, 1),        # many tiny tensors, then one that holds the tiles
    ([700001, 3, 1 << 20, 5, 1 << 21, 77, 900000, 65536, 1 << 20, 9], 5, 0, 5),  # ten uneven tensors
    ([(1 << 19) + 977 * i for i in range(20)], 15, 0, 15),  # twenty tensors: fifteen pieces
    # the same list with each pass launched in dispatches of at most 333 tiles
    ([700001, 3, 1 << 20, 5, 1 << 21, 77, 900000, 65536, 1 << 20, 9], 5, 333, 38),
])
def test_pieces_cover_every_tensor_once(torch, sizes, pieces, dispatch_tiles, dispatches):
    """However the list is cut into pieces (each at least one tensor, about
    equal tiles) and each piece's passes into dispatches, every tensor's
    values, scales and param-sync copy equal the oracle's after two steps."""
    host = host_tensors(sizes, g_dtype="bf16", p_kind="f16_scaled", p_out="bf16", seed=len(sizes),
                        m_v_init="random")
    assert sum(sizes) >= 1 << 22
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, dispatch_tiles=dispatch_tiles, scaled_passes=2))
    assert (tl.info()["pieces"], tl.info()["dispatches"]) == (pieces, dispatches)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    orc = oracle.default()
    ot, st, step = oracle_tensors(ref), [0], A.HostStep(0)
    for _ in range(2):
        A.adam_step_scaled(tl, hl, 1.6e-3, step)
        orc.group_step(ot, hr, 1.6e-3, st, 1.0)
    torch.cuda.synchronize()
    assert_bitwise(dev.readback(), ref, ctx=f"{len(sizes)} tensors")
    tl.destroy()
