"""GPU parity of the gradient sum of squares and the clip / found-inf step,
and of the whole capturable step they feed (sum -> clip -> update), through
the C ABI against the oracle."""
import gc
import zlib

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, hp_pair, oracle_tensors, torch_mod
from workloads import device_flat, host_tensors, split_views, workloads

pytestmark = pytest.mark.gpu

# The library adds squares in double in a fixed order; against the exact sum
# its relative error is bounded by (additions on the longest path) * 2^-53:
# at most about 600 here (512 squares per lane, the workgroup tree, the fold
# of the partial sums), far below this tolerance.
SUMSQ_RTOL = 1e-12


def assert_clip_from_exact_sum(orc, exact, gpu, scale0, max_norm, got_norm, got_scale, got_noop):
    """The norm, new grad scale and found-inf flag the oracle computes from
    its own exact sum of squares equal the GPU's (which started from the
    GPU's sum).  The two sums differ by at most SUMSQ_RTOL (relative), so
    their float norms can differ only when the norm of the exact sum lies
    within that window of a float rounding boundary (the square root halves
    the relative difference); then the two float norms must be neighbours
    with that boundary between them."""
    import math

    norm, new_s, found = orc.clip_grad_scale(exact, scale0, max_norm)
    same = lambda a, b: a == b or (np.isnan(a) and np.isnan(b))
    if not (math.isfinite(exact) and math.isfinite(gpu)):
        assert same(np.float32(gpu), np.float32(exact))  # both inf, or both NaN
    raw_exact = np.float32(math.sqrt(exact)) if exact == exact else np.float32(np.nan)
    raw_gpu = np.float32(math.sqrt(gpu)) if gpu == gpu else np.float32(np.nan)
    if same(raw_exact, raw_gpu):
        assert same(np.float32(got_norm), norm), (got_norm, norm)
        assert np.float32(got_scale) == new_s, (got_scale, new_s)
        assert got_noop == found
    else:
        assert np.nextafter(raw_exact, raw_gpu) == raw_gpu, (raw_exact, raw_gpu)
        boundary = (float(raw_exact) + float(raw_gpu)) / 2
        assert abs(math.sqrt(exact) - boundary) <= SUMSQ_RTOL * boundary


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


@pytest.fixture(autouse=True)
def free_memory():
    yield
    t = torch_mod()
    gc.collect()
    if t.cuda.is_available():
        t.cuda.empty_cache()


SIZES = list(range(0, 68)) + [4095, 4096, 4097, 33000, 65537, 200003]


def gpu_sumsq(torch, tl, accumulate=False, start=0.0):
    d = torch.tensor([start], dtype=torch.float64, device="cuda")
    A.adam_grad_sumsq(tl, d, accumulate)
    torch.cuda.synchronize()
    return float(d.item())


@pytest.mark.parametrize("g_dtype,p_kind,layout", [
    ("f32", "f32", "aligned"), ("bf16", "f32", "shared"), ("f32", "f32", "random"),
    ("bf16", "bf16_rem", "shared"), ("bf16", "f32", "random"), ("f16", "f32", "random"),
    ("f16", "f16_scaled", "shared")])
def test_grad_sumsq_matches_the_exact_sum(torch, orc, g_dtype, p_kind, layout):
    rng = np.random.default_rng(zlib.crc32(f"{g_dtype}{p_kind}{layout}".encode()))
    host = host_tensors(SIZES, g_dtype=g_dtype, p_kind=p_kind, seed=51)
    for h in host[::5]:  # magnitudes across many decades
        if h.g.dtype == np.float32 and h.g.size:
            h.g *= np.float32(10.0 ** rng.uniform(-20, 20))
    roles = ("p", "rem", "m", "v", "g", "p_out")
    if layout == "aligned":
        offsets = None
    elif layout == "shared":
        offsets = [{r: k % 8 for r in roles} for k in range(len(SIZES))]
    else:
        offsets = [{r: int(rng.integers(0, 8)) for r in roles} for _ in SIZES]
    dev = DeviceSet(host, offsets)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    got = gpu_sumsq(torch, tl)
    want = orc.grad_sumsq([h.g for h in host])
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)
    # deterministic, and accumulate adds to what is there
    assert gpu_sumsq(torch, tl) == got
    assert gpu_sumsq(torch, tl, True, 0.5) == 0.5 + got
    tl.destroy()


@pytest.mark.parametrize("g_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("layout,chunk", [("aligned", 0), ("aligned", 4096), ("shared", 0)])
def test_grad_sumsq_every_tail_length(torch, orc, g_dtype, layout, chunk):
    st = A.adam_tl_plan([dict(p=1 << 40, m=2 << 40, v=3 << 40, g=4 << 40, numel=8)],
                        A.make_desc(g=g_dtype))
    tile = st["tile_elems"]
    sizes = [tile + r for r in range(tile)] + [3 * tile - 1, 3 * tile - 5]
    host = host_tensors(sizes, g_dtype=g_dtype, seed=62)
    roles = ("p", "rem", "m", "v", "g", "p_out")
    offsets = None if layout == "aligned" else [{r: k % 67 for r in roles} for k in range(len(sizes))]
    dev = DeviceSet(host, offsets)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, chunk_elems=chunk))
    got = gpu_sumsq(torch, tl)
    want = orc.grad_sumsq([h.g for h in host])
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)


def test_grad_sumsq_of_an_empty_group_and_of_chained_groups(torch, orc):
    empty = A.adam_tl_build([], A.make_desc(), stream=0)
    assert gpu_sumsq(torch, empty) == 0.0
    assert gpu_sumsq(torch, empty, True, 3.25) == 3.25
    h1 = host_tensors([1000, 77], seed=52)
    h2 = host_tensors([4096 * 3 + 1], g_dtype="bf16", seed=53)
    d1, d2 = DeviceSet(h1), DeviceSet(h2)
    t1 = A.adam_tl_build(d1.tensors, desc_for(h1))
    t2 = A.adam_tl_build(d2.tensors, desc_for(h2))
    a, b = gpu_sumsq(torch, t1), gpu_sumsq(torch, t2)
    d = torch.zeros(1, dtype=torch.float64, device="cuda")
    A.adam_grad_sumsq(t1, d, False)
    A.adam_grad_sumsq(empty, d, True)
    A.adam_grad_sumsq(t2, d, True)
    torch.cuda.synchronize()
    assert float(d.item()) == a + b
    want = orc.grad_sumsq([h.g for h in h1] + [h.g for h in h2])
    assert abs(a + b - want) <= SUMSQ_RTOL * want


def test_grad_sumsq_of_non_finite_gradients(torch):
    host = host_tensors([5000, 300], seed=54)
    host[0].g[1234] = np.inf
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    assert gpu_sumsq(torch, tl) == np.inf
    dev.tensors[1]["g"][5] = float("nan")
    assert np.isnan(gpu_sumsq(torch, tl))


@pytest.mark.parametrize("case", ["clip", "no_clip", "max_norm_zero", "inf", "nan"])
def test_clip_grad_scale_equals_the_oracle_bitwise(torch, orc, case):
    host = host_tensors([30000, 513], g_dtype="bf16", seed=55)
    if case == "inf":
        host[1].g[7] = 0x7F80  # bf16 +inf
    if case == "nan":
        host[0].g[9] = 0x7FC0
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    A.adam_grad_sumsq(tl, d_sumsq, False)
    scale0 = 0.37
    max_norm = {"clip": 1e-3, "no_clip": 1e6, "max_norm_zero": 0.0}.get(case, 1.0)
    d_scale = torch.tensor([scale0], dtype=torch.float32, device="cuda")
    d_norm = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_noop = torch.tensor([1], dtype=torch.int32, device="cuda")  # overwritten either way
    A.adam_clip_grad_scale(d_sumsq, d_scale, max_norm, d_norm, d_noop)
    torch.cuda.synchronize()
    norm, new_s, found = orc.clip_grad_scale(float(d_sumsq.item()), np.float32(scale0), max_norm)
    got_norm = np.float32(d_norm.item())
    assert (got_norm == norm) or (np.isnan(got_norm) and np.isnan(norm))
    assert np.float32(d_scale.item()) == new_s
    assert int(d_noop.item()) == found == (1 if case in ("inf", "nan") else 0)
    # the same from the oracle's own exact sum of the gradients
    exact = orc.grad_sumsq([h.g for h in host])
    assert_clip_from_exact_sum(orc, exact, float(d_sumsq.item()), np.float32(scale0), max_norm,
                               got_norm, d_scale.item(), int(d_noop.item()))
    if case == "clip":
        assert new_s < np.float32(scale0)
    if case in ("no_clip", "max_norm_zero", "inf", "nan"):
        assert new_s == np.float32(scale0)


def test_clip_argument_errors(torch):
    L = A.lib()
    d = torch.zeros(1, dtype=torch.float64, device="cuda")
    assert L.adam_clip_grad_scale(None, None, 0.0, None, None, None) == A.ADAM_EINVAL
    assert L.adam_clip_grad_scale(d.data_ptr(), None, 1.0, None, None, None) == A.ADAM_EINVAL
    assert L.adam_clip_grad_scale(d.data_ptr(), None, float("nan"), None, None, None) == A.ADAM_EINVAL
    tl = A.adam_tl_build([], A.make_desc(), stream=0)
    assert L.adam_grad_sumsq(tl.handle, None, 0, None) == A.ADAM_EINVAL
    assert L.adam_grad_sumsq(tl.handle, d.data_ptr(), 2, None) == A.ADAM_EINVAL
    assert L.adam_grad_sumsq(None, d.data_ptr(), 0, None) == A.ADAM_EINVAL


@pytest.mark.parametrize("g_dtype,p_kind,p_out,two_buffer",
                         [("bf16", "f32", "bf16", False), ("bf16", "bf16_rem", "bf16", False),
                          ("f16", "f32", "f16", False), ("bf16", "f16_scaled", "f16", False),
                          ("bf16", "f32", "bf16", True), ("bf16", "bf16_rem", "bf16", True)])
def test_whole_capturable_step_in_one_graph(torch, orc, g_dtype, p_kind, p_out, two_buffer):
    """Two groups (decay and no decay): per step the gradient sum of squares
    of both groups, the clip / found-inf step, then the capturable update of
    each group (fp32 master, bf16 + remainders, or scaled fp16 state; also
    with the state in two buffer sets), all recorded in one HIP graph and
    replayed; an infinite gradient on the third replay skips that step.
    Each replay equals the oracle fed the same sum of squares; with two
    buffer sets the four steps taken leave the state in the first set."""
    h1 = host_tensors([40000, 4096, 333], g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=56)
    h2 = host_tensors([4096] * 3, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=57)
    cap = {"bf16_rem": A.adam_step_remainders_capturable,
           "f16_scaled": A.adam_step_scaled_capturable}.get(p_kind, A.adam_step_capturable)
    d1, d2 = DeviceSet(h1), DeviceSet(h2)
    if two_buffer:
        keep = []

        def second(dev):
            alts = [{r: torch.full_like(t[r], 7) for r in ("p", "m", "v", "rem") if r in t} for t in dev.tensors]
            keep.append(alts)
            return alts

        t1 = A.adam_tl_build(d1.tensors, desc_for(h1), alternates=second(d1))
        t2 = A.adam_tl_build(d2.tensors, desc_for(h2), alternates=second(d2))
    else:
        t1 = A.adam_tl_build(d1.tensors, desc_for(h1))
        t2 = A.adam_tl_build(d2.tensors, desc_for(h2))
    hp1, hr1 = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    hp2, hr2 = hp_pair(0.9, 0.95, 1e-8, 0.0, 1)
    d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
    d_scale = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    d_sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    d_norm = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    s1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    s2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    max_norm = 0.05

    def step(stream):
        A.adam_grad_sumsq(t1, d_sumsq, False, stream)
        A.adam_grad_sumsq(t2, d_sumsq, True, stream)
        A.adam_clip_grad_scale(d_sumsq, d_scale, max_norm, d_norm, d_noop, stream)
        cap(t1, hp1, d_lr, s1, d_scale, d_noop, stream)
        cap(t2, hp2, d_lr, s2, d_scale, d_noop, stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    assert int(s1.item()) == 0  # capture records, does not run

    r1, r2 = oracle_tensors(copies(h1)), oracle_tensors(copies(h2))
    st1, st2 = [0], [0]
    for k in range(5):
        d_scale.fill_(1.0)  # the optimizer resets its grad scale every iteration
        if k == 2:
            d1.tensors[0]["g"][11] = float("inf")
        graph.replay()
        torch.cuda.synchronize()
        sumsq = float(d_sumsq.item())
        want = orc.grad_sumsq([t.g for t in r1] + [t.g for t in r2])
        if k == 2:
            assert sumsq == np.inf and int(d_noop.item()) == 1
            d1.tensors[0]["g"][11] = 0.0
            r1[0].g[11] = 0
        else:
            assert abs(sumsq - want) <= SUMSQ_RTOL * want
        norm, new_s, found = orc.clip_grad_scale(sumsq, 1.0, max_norm)
        assert np.float32(d_norm.item()) == norm or (np.isnan(norm) and np.isnan(d_norm.item()))
        assert np.float32(d_scale.item()) == new_s
        # the same from the oracle's own exact sum (on the replay with the
        # injected inf, the oracle's copy of the gradients does not hold it)
        if k != 2:
            assert_clip_from_exact_sum(orc, want, sumsq, 1.0, max_norm, d_norm.item(), d_scale.item(),
                                       int(d_noop.item()))
        orc.group_step(r1, hr1, 1.6e-3, st1, float(new_s), noop=found)
        orc.group_step(r2, hr2, 1.6e-3, st2, float(new_s), noop=found)
    assert int(s1.item()) == st1[0] == 4 and int(s2.item()) == st2[0] == 4
    assert_bitwise(d1.readback(), r1, ctx="group 1")
    assert_bitwise(d2.readback(), r2, ctx="group 2")


def test_grad_sumsq_full_size_201_tensors(torch, orc):
    """4,215,275,520 fp32 gradients (the benchmark's list): against the exact
    sum (gradients copied to the host in 1 GiB pieces), repeatable bit for
    bit, and exactly 4x after doubling every gradient (a power-of-two scale
    commutes with every rounding)."""
    w = workloads()["bench201"]
    bufs = device_flat(w.numel, g_dtype="f32", p_kind="f32", p_out=False, seed=w.seed)
    views = {k: split_views(v, w.sizes) for k, v in bufs.items()}
    tensors = [{k: views[k][i] for k in views} for i in range(len(w.sizes))]
    tl = A.adam_tl_build(tensors, A.make_desc())
    got = gpu_sumsq(torch, tl)
    assert gpu_sumsq(torch, tl) == got
    total = orc.new_accumulator()
    piece = 1 << 28
    for lo in range(0, w.numel, piece):
        host = bufs["g"][lo:lo + piece].cpu().numpy()
        orc.accumulate_squares(total, [host], threads=16)
        del host
    want = orc.accumulator_value(total)
    assert abs(got - want) <= SUMSQ_RTOL * want, (got, want)
    bufs["g"].mul_(2.0)
    assert gpu_sumsq(torch, tl) == 4.0 * got
    tl.destroy()
