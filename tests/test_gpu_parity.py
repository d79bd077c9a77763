"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs (sizes the oracle finishes in seconds, spanning
several work items, tiles and ragged tails), plus the self-consistency
properties of the capturable, graph and remainder paths."""
import zlib

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import (DeviceSet, assert_bitwise, assert_within_tolerance, copies, desc_for,
                         hp_pair, oracle_tensors, torch_mod)
from workloads import TINY_SIZES, host_tensors, workloads

pytestmark = pytest.mark.gpu


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


def run_both(orc, host, hp_lib, hp_ref, lr, steps, *, grad_scale=1.0, desc_kw=None, offsets=None,
             remainder=None):
    """Runs `steps` non-capturable steps on the GPU and on the oracle from the
    same inputs; returns (gpu result, oracle result, gpu step, oracle step)."""
    torch = torch_mod()
    ref = copies(host)
    dev = DeviceSet(host, offsets)
    desc = desc_for(host, **(desc_kw or {}))
    tl = A.adam_tl_build(dev.tensors, desc)
    rem = host[0].rem is not None if remainder is None else remainder
    fn = A.adam_step_remainders if rem else A.adam_step
    if host[0].scales is not None:
        fn = A.adam_step_scaled
    step = A.HostStep(0)
    ref_step = [0]
    ot = oracle_tensors(ref)
    for _ in range(steps):
        fn(tl, hp_lib, lr, step, grad_scale)
        orc.group_step(ot, hp_ref, lr, ref_step, grad_scale)
    torch.cuda.synchronize()
    got = dev.readback()
    tl.destroy()
    return got, ref, step.value, ref_step[0]


def test_tiny_case_l2_and_adamw_ten_steps(torch, orc):
    """Three fp32 tensors (4096, 1000, 7), p ~ N(0,1), g ~ N(0,1)*1e-3 drawn
    once, lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.01; ten steps in L2 mode
    and, from the same start, ten in AdamW mode."""
    w = workloads()["tiny"]
    host = host_tensors(TINY_SIZES, seed=w.seed)
    for mode in (0, 1):
        hl, hr = hp_pair(w.beta1, w.beta2, w.eps, w.weight_decay, mode)
        got, ref, s, rs = run_both(orc, host, hl, hr, w.lr, 10)
        assert s == rs == 10
        assert_within_tolerance(got, ref)
        assert_bitwise(got, ref, ctx=f"mode {mode}")


SWEEP_SIZES = list(range(0, 68)) + [4095, 4096, 4097, 4096 * 3 + 5, 10000, 65537]


@pytest.mark.parametrize("g_dtype,p_kind,p_out,mode", [
    ("f32", "f32", False, 0), ("f32", "f32", False, 1), ("bf16", "f32", False, 1),
    ("bf16", "f32", True, 0), ("f32", "f32", True, 1), ("bf16", "bf16_rem", False, 1),
    ("f32", "bf16_rem", True, 0), ("bf16", "bf16_rem", True, 1), ("f16", "f32", "f16", 1),
    ("f16", "bf16_rem", True, 0), ("bf16", "f16_scaled", "f16", 1), ("f32", "f16_scaled", False, 0),
    ("f16", "bf16_scaled", "bf16", 1), ("bf16", "bf16", True, 1), ("f32", "f16", "f32", 0),
    ("f16", "f16", "bf16", 1), ("bf16", "bf16", "f16", 0), ("f32", "f32", "f32", 1), ("bf16", "f16", False, 1)])
def test_tail_and_offset_sweep(torch, orc, g_dtype, p_kind, p_out, mode):
    """Every size 0..67 plus sizes around and across work-item boundaries, with
    each buffer of each tensor at its own element offset 0..7 (so some tensors
    take the 4-element path and some the element path), three steps,
    bitwise against the oracle."""
    rng = np.random.default_rng(zlib.crc32(f"{g_dtype}{p_kind}{p_out}{mode}".encode()))
    host = host_tensors(SWEEP_SIZES, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=7,
                        m_v_init="large" if p_kind == "bf16_scaled" else "random")
    offsets = []
    for i in range(len(SWEEP_SIZES)):
        if i % 3 == 0:
            offsets.append({})  # aligned
        else:
            offsets.append({r: int(rng.integers(0, 8)) for r in ("p", "rem", "m", "v", "g", "p_out")})
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref, s, rs = run_both(orc, host, hl, hr, 1.6e-3, 3, grad_scale=0.5,
                               desc_kw=dict(chunk_elems=4096), offsets=offsets)
    assert s == rs == 3
    assert_bitwise(got, ref, ctx=f"{g_dtype}/{p_kind}/{p_out}/{mode}")


@pytest.mark.parametrize("g_dtype,p_kind,p_out,mode", [
    ("f32", "f32", False, 1), ("bf16", "f32", True, 0), ("bf16", "bf16_rem", False, 1),
    ("f32", "bf16_rem", True, 1), ("f16", "f32", "f16", 1), ("bf16", "f16_scaled", "bf16", 0),
    ("bf16", "bf16", True, 1), ("f16", "f16", "f32", 0), ("f32", "f32", "f32", 1)])
def test_shared_offsets_take_the_peeled_vector_path(torch, orc, g_dtype, p_kind, p_out, mode):
    """Every stream of a tensor at the same element offset 0..7 (views at one
    offset into flat buffers): the leading elements before the first lane
    group boundary (or 128-byte line) are peeled and the rest vectorised;
    results stay bit-identical to the oracle."""
    sizes = list(range(0, 20)) + [1021, 4095, 4099, 8193, 70001]
    host = host_tensors(sizes, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=31,
                        m_v_init="random")
    roles = ("p", "rem", "m", "v", "g", "p_out")
    offsets = [{r: k % 8 for r in roles} for k in range(len(sizes))]
    desc = desc_for(host, chunk_elems=4096)
    dev = DeviceSet(host, offsets)
    st = A.adam_tl_build(dev.tensors, desc).info()
    lane = st["tile_elems"] // st["block_threads"]
    assert st["vector_tensors"] == sum(1 for k, n in enumerate(sizes) if n > (lane - k % lane) % lane)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref, s, rs = run_both(orc, host, hl, hr, 1.6e-3, 3, grad_scale=0.5,
                               desc_kw=dict(chunk_elems=4096), offsets=offsets)
    assert s == rs == 3
    assert_bitwise(got, ref, ctx=f"{g_dtype}/{p_kind}/{p_out}/{mode}")


def tile_elems(g_dtype="f32", p_kind="f32", p_out=False):
    """Elements per workgroup tile of a list with these dtypes (planned on
    fake addresses, nothing is dereferenced)."""
    t = dict(p=1 << 40, m=2 << 40, v=3 << 40, g=4 << 40, numel=8)
    if p_kind == "bf16_rem":
        t["rem"] = 5 << 40
    if p_kind.endswith("_scaled"):
        t["scales"] = 7 << 40
    if p_out:
        t["p_out"] = 6 << 40
    desc = A.make_desc(g=g_dtype, p=p_kind, p_out=("bf16" if p_out is True else p_out) or None)
    return A.adam_tl_plan([t], desc)["tile_elems"]


@pytest.mark.parametrize("g_dtype,p_kind,p_out", [
    ("f32", "f32", False), ("bf16", "f32", True), ("bf16", "bf16_rem", False), ("f16", "f32", "f16"),
    ("bf16", "f16_scaled", "f16"), ("bf16", "bf16", True), ("f16", "f16", "f32")])
@pytest.mark.parametrize("layout,chunk", [("aligned", 0), ("aligned", 4096), ("shared", 0)])
def test_every_tail_length(torch, orc, g_dtype, p_kind, p_out, layout, chunk):
    """One tensor per tail length: a full tile plus 0..tile-1 elements, so the
    last tile of every vector body takes every possible ragged length
    (including the ones whose tail lanes follow the last vector lane)."""
    tile = tile_elems(g_dtype, p_kind, p_out)
    sizes = [tile + r for r in range(tile)] + [3 * tile - 1, 3 * tile - 2, 3 * tile - 5]
    host = host_tensors(sizes, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=61,
                        m_v_init="random")
    roles = ("p", "rem", "m", "v", "g", "p_out")
    offsets = None if layout == "aligned" else [{r: k % 67 for r in roles} for k in range(len(sizes))]
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref, s, rs = run_both(orc, host, hl, hr, 1.6e-3, 2, desc_kw=dict(chunk_elems=chunk),
                               offsets=offsets)
    assert s == rs == 2
    assert_bitwise(got, ref, ctx=f"{g_dtype}/{p_kind}/{p_out}/{layout}/{chunk}")


def test_results_do_not_depend_on_chunk(torch, orc):
    sizes = [70001, 4096 * 5, 123, 9, 65536 * 2]
    host = host_tensors(sizes, g_dtype="bf16", p_out=True, seed=21, m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    results = []
    for kw in (dict(chunk_elems=1024), dict(chunk_elems=4096), dict(chunk_elems=65536),
               dict(chunk_elems=1 << 20), dict()):
        got, ref, _, _ = run_both(orc, host, hl, hr, 1.6e-3, 2, desc_kw=kw)
        assert_bitwise(got, ref, ctx=str(kw))
        results.append(got)
    for r in results[1:]:
        assert_bitwise(r, results[0])


@pytest.mark.parametrize("g_dtype,p_kind,p_out,mode,dispatch_tiles", [
    ("f32", "f32", False, 1, 1), ("bf16", "f32", True, 0, 3), ("bf16", "bf16_rem", True, 1, 7),
    ("f16", "bf16", "f32", 1, 64), ("bf16", "f16_scaled", "bf16", 1, 5), ("f32", "f32", "f32", 0, 513)])
def test_split_dispatches_match_the_oracle(torch, orc, g_dtype, p_kind, p_out, mode, dispatch_tiles):
    """A list launched as many dispatches of at most `dispatch_tiles` tiles
    (the way lists beyond one dispatch's 32-bit work-item count run): host
    steps, then capturable steps, bitwise against the oracle."""
    sizes = SWEEP_SIZES
    host = host_tensors(sizes, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=43, m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, chunk_elems=4096, dispatch_tiles=dispatch_tiles))
    info = tl.info()
    assert info["dispatch_tiles"] == dispatch_tiles
    assert info["dispatches"] == -(-info["grid_blocks"] // dispatch_tiles) > 1
    scaled = host[0].scales is not None
    host_fn = (A.adam_step_scaled if scaled else A.adam_step_remainders if host[0].rem is not None
               else A.adam_step)
    cap_fn = (A.adam_step_scaled_capturable if scaled else A.adam_step_remainders_capturable
              if host[0].rem is not None else A.adam_step_capturable)
    ref = copies(host)
    ot, st, step = oracle_tensors(ref), [0], A.HostStep(0)
    for _ in range(2):
        host_fn(tl, hl, 1.6e-3, step, 0.5)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5)
    torch.cuda.synchronize()
    assert_bitwise(dev.readback(), ref, ctx=f"host steps, {info['dispatches']} dispatches")
    d_lr = torch.tensor([1.6e-3], dtype=torch.float32, device="cuda")
    d_step = torch.tensor([st[0]], dtype=torch.int32, device="cuda")
    d_s = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    for _ in range(2):
        cap_fn(tl, hl, d_lr, d_step, d_s, None)
        orc.group_step(ot, hr, 1.6e-3, st, 0.5)
    torch.cuda.synchronize()
    assert int(d_step.item()) == st[0] == 4
    assert_bitwise(dev.readback(), ref, ctx=f"capturable steps, {info['dispatches']} dispatches")
    tl.destroy()


def test_device_grad_scale_equals_host_grad_scale(torch, orc):
    host = host_tensors([5000, 333], seed=22)
    hl, hr = hp_pair(0.9, 0.999, 1e-8, 0.01, 0)
    outs = []
    for use_dev in (False, True):
        dev = DeviceSet(host)
        tl = A.adam_tl_build(dev.tensors, desc_for(host))
        d_s = torch.tensor([0.25], dtype=torch.float32, device="cuda")
        step = A.HostStep(0)
        for _ in range(3):
            if use_dev:
                A.adam_step(tl, hl, 1e-3, step, grad_scale=123.0, d_grad_scale=d_s)
            else:
                A.adam_step(tl, hl, 1e-3, step, grad_scale=0.25)
        torch.cuda.synchronize()
        outs.append(dev.readback())
    assert_bitwise(outs[1], outs[0])
    ref = copies(host)
    ot = oracle_tensors(ref)
    st = [0]
    for _ in range(3):
        orc.group_step(ot, hr, 1e-3, st, 0.25)
    assert_bitwise(outs[0], ref)


def _capturable_setup(torch, host, lr=1.6e-3, scale=1.0, step0=0):
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr = torch.tensor([lr], dtype=torch.float32, device="cuda")
    d_step = torch.tensor([step0], dtype=torch.int32, device="cuda")
    d_s = torch.tensor([scale], dtype=torch.float32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    return dev, tl, d_lr, d_step, d_s, d_noop


@pytest.mark.parametrize("g_dtype,p_out,mode", [("f32", False, 1), ("bf16", True, 1), ("f32", True, 0)])
def test_capturable_equals_noncapturable_and_oracle(torch, orc, g_dtype, p_out, mode):
    host = host_tensors([20000, 4097, 64, 3], g_dtype=g_dtype, p_out=p_out, seed=23)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    dev, tl, d_lr, d_step, d_s, d_noop = _capturable_setup(torch, host, scale=0.5)
    for _ in range(5):
        A.adam_step_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 5
    got_c = dev.readback()
    got_n, ref, s, rs = run_both(orc, host, hl, hr, 1.6e-3, 5, grad_scale=0.5)
    assert s == rs == 5
    assert_bitwise(got_c, got_n, ctx="capturable vs non-capturable")
    assert_bitwise(got_c, ref, ctx="capturable vs oracle")


def test_noop_flag_leaves_every_buffer_and_the_counter(torch, orc):
    host = host_tensors([10000, 77], g_dtype="bf16", p_out=True, seed=24, m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    dev, tl, d_lr, d_step, d_s, d_noop = _capturable_setup(torch, host, step0=4)
    # a p_out that is not yet the cast of p, so a stray write would show
    for d in dev.tensors:
        d["p_out"].fill_(7.0)
    before = dev.readback()
    d_noop.fill_(1)
    dev.set_grad(0, 17, float("inf"))
    for _ in range(3):
        A.adam_step_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 4
    after = dev.readback()
    for b, a in zip(before, after):
        for r in ("p", "m", "v", "p_out"):
            assert np.array_equal(getattr(b, r).view(np.uint8), getattr(a, r).view(np.uint8)), r
    # flag values other than 1 run the step
    dev.set_grad(0, 17, 0.0)
    d_noop.fill_(2)
    A.adam_step_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 5
    # and the result is the oracle's step 5 from the state left at step 4
    ref = copies(before)
    ref[0].g[17] = 0
    ot = oracle_tensors(ref)
    st = [4]
    orc.group_step(ot, hr, 1.6e-3, st, 1.0, noop=2)
    assert_bitwise(dev.readback(), ref)


def test_empty_group_counter_advances_on_device(torch):
    """A handle with no elements: the capturable call still advances the
    device counter (three steps -> 3), and not when the flag is 1."""
    tl = A.adam_tl_build([], A.make_desc(), stream=0)
    hl, _ = hp_pair()
    d_lr = torch.tensor([1e-3], device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        A.adam_step_capturable(tl, hl, d_lr, d_step, None, d_noop)
    d_noop.fill_(1)
    A.adam_step_capturable(tl, hl, d_lr, d_step, None, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 3
    A.adam_step_capturable(tl, hl, d_lr, d_step, None, None)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 4


def test_graph_replay_equals_eager(torch, orc):
    """One capturable step captured into a HIP graph and replayed five times
    (with eager work and synchronisation between replays, and lr changed on
    the device between replays) equals five eager capturable steps."""
    host = host_tensors([50000, 4096, 13], g_dtype="bf16", p_out=True, seed=25)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    lrs = [1e-3, 2e-3, 5e-4, 1e-3, 3e-3]

    dev_e, tl_e, lr_e, st_e, s_e, n_e = _capturable_setup(torch, host)
    for lr in lrs:
        lr_e.fill_(lr)
        A.adam_step_capturable(tl_e, hl, lr_e, st_e, s_e, n_e)
    torch.cuda.synchronize()
    eager = dev_e.readback()

    dev_g, tl_g, lr_g, st_g, s_g, n_g = _capturable_setup(torch, host)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        A.adam_step_capturable(tl_g, hl, lr_g, st_g, s_g, n_g)
    torch.cuda.synchronize()
    # capture recorded the step without running it
    assert int(st_g.item()) == 0
    for lr in lrs:
        lr_g.fill_(lr)
        graph.replay()
        torch.cuda.synchronize()
        _ = (lr_g * 2).sum().item()  # unrelated eager work between replays
    assert int(st_g.item()) == 5
    assert_bitwise(dev_g.readback(), eager, ctx="graph vs eager")
    # and both equal the oracle with the same lr schedule
    ref = copies(host)
    ot = oracle_tensors(ref)
    st = [0]
    for lr in lrs:
        orc.group_step(ot, hr, lr, st, 1.0, noop=0)
    assert_bitwise(eager, ref, ctx="eager vs oracle")


def test_remainder_mode_equals_fp32_mode_on_decoded_masters(torch, orc):
    """Remainder-mode results, decoded, equal the fp32 path run on the decoded
    masters (both on the GPU), bit for bit; and p_out is the stored bf16."""
    host = host_tensors([30001, 4096, 5], g_dtype="bf16", p_kind="bf16_rem", p_out=True, seed=26,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got_r, ref_r, _, _ = run_both(orc, host, hl, hr, 1.6e-3, 4)
    assert_bitwise(got_r, ref_r, ctx="remainder vs oracle")
    masters = [orc.rem_decode(h.p, h.rem) for h in host]
    host32 = copies(host)
    for h, mstr in zip(host32, masters):
        h.p, h.rem, h.p_out = mstr, None, None
    got_f, _, _, _ = run_both(orc, host32, hl, hr, 1.6e-3, 4)
    for r, f in zip(got_r, got_f):
        dec = orc.rem_decode(r.p, r.rem)
        assert np.array_equal(dec.view(np.uint32), f.p.view(np.uint32))
        assert np.array_equal(r.m.view(np.uint32), f.m.view(np.uint32))
        assert np.array_equal(r.p_out, r.p)


def test_nonfinite_gradient_propagates_without_noop(torch, orc):
    host = host_tensors([4096, 100], seed=27)
    host[0].g[[3, 4000]] = [np.inf, np.nan]
    host[1].g[99] = -np.inf
    hl, hr = hp_pair(0.9, 0.999, 1e-8, 0.01, 1)
    got, ref, _, _ = run_both(orc, host, hl, hr, 1e-3, 2)
    assert_bitwise(got, ref)
    assert not np.isfinite(got[0].p[3]) and not np.isfinite(got[1].p[99])
    assert np.isfinite(np.delete(got[0].p, [3, 4000])).all()


def test_bias_correction_off_and_extreme_hyperparameters(torch, orc):
    host = host_tensors([9000, 31], g_dtype="bf16", seed=28, m_v_init="random")
    for hp in [(0.9, 0.999, 1e-8, 0.0, 1, 0), (0.5, 0.5, 1e-2, 0.5, 0, 1),
               (0.0, 0.0, 1e-12, 0.1, 1, 1), (0.99, 0.9999, 1e-8, 0.01, 0, 0)]:
        hl, hr = hp_pair(*hp)
        got, ref, _, _ = run_both(orc, host, hl, hr, 3e-2, 6, grad_scale=2.0 ** -10)
        assert_bitwise(got, ref, ctx=str(hp))


def test_subnormal_values_are_kept(torch, orc):
    """fp32 denormals in p, g and the moments are not flushed (in AdamW mode
    a denormal gradient leaves a denormal first moment)."""
    host = host_tensors([4096], seed=29)
    host[0].g[:64] = np.float32(1e-41)
    host[0].p[64:128] = np.float32(-3e-40)
    host[0].m[128:192] = np.float32(2e-39)
    host[0].v[128:192] = np.float32(1e-40)
    for mode in (0, 1):
        hl, hr = hp_pair(0.9, 0.999, 1e-30, 0.01, mode)
        got, ref, _, _ = run_both(orc, host, hl, hr, 1e-3, 3, grad_scale=0.75)
        assert_bitwise(got, ref, ctx=f"mode {mode}")
        if mode == 1:
            m = np.abs(got[0].m[:64])
            assert np.all((m > 0) & (m < np.finfo(np.float32).tiny))
