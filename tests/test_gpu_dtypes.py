"""GPU parity of the rest of the dtype matrix and of scaled optimizer state,
through the C ABI against the oracle: fp16 gradients and fp16 param-out,
the capturable remainder step, and per-tensor scaled 16-bit p / m / v
(apex distributed_fused_adam.py, _local_step_with_scaled_states and
_apply_state_scale).  Bit-for-bit, NaN compared as NaN."""
import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import (DeviceSet, assert_bitwise, assert_within_tolerance, copies, desc_for,
                         hp_pair, oracle_tensors, torch_mod)
from workloads import host_tensors

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


def run_steps(orc, host, hl, hr, lr, steps, *, grad_scale=1.0, desc_kw=None, offsets=None):
    """`steps` non-capturable steps on the GPU (the step call the handle's
    storage needs) and on the oracle from the same inputs."""
    torch = torch_mod()
    ref = copies(host)
    dev = DeviceSet(host, offsets)
    tl = A.adam_tl_build(dev.tensors, desc_for(host, **(desc_kw or {})))
    h = host[0]
    fn = A.adam_step_scaled if h.scales is not None else \
        A.adam_step_remainders if h.rem is not None else A.adam_step
    step, ref_step = A.HostStep(0), [0]
    ot = oracle_tensors(ref)
    for _ in range(steps):
        fn(tl, hl, lr, step, grad_scale)
        orc.group_step(ot, hr, lr, ref_step, grad_scale)
    torch.cuda.synchronize()
    got = dev.readback()
    tl.destroy()
    assert step.value == ref_step[0] == steps
    return got, ref


SIZES = [0, 1, 3, 4, 5, 63, 64, 65, 511, 512, 513, 4095, 4097, 20001, 70001]


# ---------------------------------------------------------------------------
# fp16 gradients and param-out
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p_kind,p_out,mode", [("f32", "f16", 1), ("f32", "f16", 0),
                                               ("f32", "bf16", 1), ("bf16_rem", True, 1)])
def test_fp16_gradients_match_the_oracle(torch, orc, p_kind, p_out, mode):
    """fp16 gradients (with subnormal, large and signed-zero values) into fp32
    or remainder params; fp16 param-out includes params beyond the fp16 range
    (infinity), at the overflow threshold, and subnormal in fp16."""
    host = host_tensors(SIZES, g_dtype="f16", p_kind=p_kind, p_out=p_out, seed=71,
                        m_v_init="random")
    big = host[-1]
    big.g[:6] = np.array([6e-8, -6e-8, 1e-5, 60000.0, -0.0, 3e-5], np.float16)
    if p_kind == "f32":
        big.p[:8] = np.array([70000.0, -70000.0, 65519.0, 65520.0, 1e-6, -3e-8, 2.0 ** -20, 65504.0],
                             np.float32)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 4, grad_scale=0.5, desc_kw=dict(chunk_elems=4096))
    assert_within_tolerance(got, ref)
    assert_bitwise(got, ref, ctx=f"{p_kind}/{p_out}/{mode}")


def test_fp16_param_out_is_the_cast_of_the_new_param(torch, orc):
    host = host_tensors([30000, 77], g_dtype="bf16", p_out="f16", seed=72)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
    assert_bitwise(got, ref)
    for t in got:
        assert np.array_equal(t.p_out.view(np.uint16), t.p.astype(np.float16).view(np.uint16))


def test_fp16_casts_through_the_update(torch, orc):
    """The fp16 conversions over many inputs, through the update itself.
    (1) p_out: with g = m = v = 0, lr = 0 and no decay the new param is the
    old one (finite p), so p_out is the fp16 cast of 2^24 random float32
    patterns from the cast's whole range (2^-26 .. 2^17 in magnitude) plus its
    edges; it must equal numpy's cast.  (2) gradients: with beta1 = 0 and
    grad scale 1 the new first moment is the widened gradient, for all 65536
    fp16 patterns.  Both also match the oracle bit for bit."""
    rng = np.random.default_rng(81)
    lo, hi = np.float32(2.0 ** -26).view(np.uint32), np.float32(2.0 ** 17).view(np.uint32)
    pats = rng.integers(int(lo), int(hi), size=1 << 24, dtype=np.int64).astype(np.uint32)
    pats[: 1 << 23] |= np.uint32(0x80000000)
    edges = np.array([65504.0, 65519.996, 65520.0, 65536.0, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25,
                      3 * 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0, -0.0], np.float32)
    p = np.concatenate([pats.view(np.float32), edges, -edges])
    n = p.size
    from workloads import HostTensor

    host = [HostTensor(p.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                       np.zeros(n, np.float16), np.zeros(n, np.float16))]
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.0, 1)
    got, ref = run_steps(orc, host, hl, hr, 0.0, 1)
    assert_bitwise(got, ref)
    assert np.array_equal(got[0].p.view(np.uint32), p.view(np.uint32))
    with np.errstate(over="ignore"):
        want = p.astype(np.float16)
    assert np.array_equal(got[0].p_out.view(np.uint16), want.view(np.uint16))
    # gradients: every fp16 pattern
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    host = [HostTensor(np.zeros(65536, np.float32), np.zeros(65536, np.float32),
                       np.zeros(65536, np.float32), g.copy())]
    hl, hr = hp_pair(0.0, 0.95, 1e-8, 0.0, 1)
    got, ref = run_steps(orc, host, hl, hr, 0.0, 1)
    assert_bitwise(got, ref)
    wide = g.astype(np.float32)
    ok = ~np.isnan(wide) & (wide != 0)
    assert np.array_equal(got[0].m[ok].view(np.uint32), wide[ok].view(np.uint32))


# ---------------------------------------------------------------------------
# Capturable remainder step
# ---------------------------------------------------------------------------

def _device_scalars(torch, lr=1.6e-3, scale=1.0, step0=0):
    return (torch.tensor([lr], dtype=torch.float32, device="cuda"),
            torch.tensor([step0], dtype=torch.int32, device="cuda"),
            torch.tensor([scale], dtype=torch.float32, device="cuda"),
            torch.zeros(1, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("g_dtype,p_out", [("bf16", True), ("f32", False), ("f16", True)])
def test_remainders_capturable_equals_noncapturable_and_oracle(torch, orc, g_dtype, p_out):
    host = host_tensors([20000, 4097, 64, 3], g_dtype=g_dtype, p_kind="bf16_rem", p_out=p_out,
                        seed=73, m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr, d_step, d_s, d_noop = _device_scalars(torch, scale=0.5)
    for _ in range(5):
        A.adam_step_remainders_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 5
    got_c = dev.readback()
    got_n, ref = run_steps(orc, host, hl, hr, 1.6e-3, 5, grad_scale=0.5)
    assert_bitwise(got_c, got_n, ctx="capturable vs non-capturable")
    assert_bitwise(got_c, ref, ctx="capturable vs oracle")


def test_remainders_capturable_noop_and_graph_replay(torch, orc):
    """The noop flag leaves bf16 params, remainders, moments, p_out and the
    counter untouched; a captured step replayed with a changing device lr
    equals the oracle's steps."""
    host = host_tensors([50000, 4096, 13], g_dtype="bf16", p_kind="bf16_rem", p_out=True, seed=74,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr, d_step, d_s, d_noop = _device_scalars(torch)
    for d in dev.tensors:
        d["p_out"].fill_(7.0)
    before = dev.readback()
    d_noop.fill_(1)
    A.adam_step_remainders_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 0
    after = dev.readback()
    for b, a in zip(before, after):
        for r in ("p", "rem", "m", "v", "p_out"):
            assert np.array_equal(getattr(b, r).view(np.uint8), getattr(a, r).view(np.uint8)), r
    d_noop.fill_(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        A.adam_step_remainders_capturable(tl, hl, d_lr, d_step, d_s, d_noop)
    torch.cuda.synchronize()
    lrs = [1e-3, 2e-3, 5e-4]
    for lr in lrs:
        d_lr.fill_(lr)
        graph.replay()
        torch.cuda.synchronize()
    assert int(d_step.item()) == 3
    ref = copies(host)
    ot = oracle_tensors(ref)
    st = [0]
    for lr in lrs:
        orc.group_step(ot, hr, lr, st, 1.0, noop=0)
    assert_bitwise(dev.readback(), ref, ctx="graph vs oracle")


# ---------------------------------------------------------------------------
# Scaled 16-bit optimizer state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p_kind,g_dtype,p_out,mode", [
    ("f16_scaled", "bf16", "bf16", 1), ("f16_scaled", "f32", None, 0), ("f16_scaled", "f16", "f16", 1),
    ("bf16_scaled", "bf16", "f16", 1), ("bf16_scaled", "f32", "bf16", 0)])
@pytest.mark.parametrize("chunk", [0, 1024])
def test_scaled_state_matches_the_oracle(torch, orc, p_kind, g_dtype, p_out, mode, chunk):
    """Several steps from a mid-training state: p, m, v (16-bit), the three
    scales of every tensor and the param-sync copy, bit for bit.  Tensors span
    many work items (so the per-tensor maxima fold across workgroups), ragged
    tails and empty tensors (whose scales stay)."""
    init = "large" if p_kind == "bf16_scaled" else "random"
    g_std = 1.0 if p_kind == "bf16_scaled" else 1e-3
    host = host_tensors(SIZES, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=75,
                        m_v_init=init, g_std=g_std)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 4, desc_kw=dict(chunk_elems=chunk))
    assert_bitwise(got, ref, ctx=f"{p_kind}/{g_dtype}/{p_out}/{mode}/{chunk}")
    for t in got[1:]:
        assert np.all(np.isfinite(t.scales)) and np.all(t.scales > 0)


def test_scaled_state_from_zero_moments(torch, orc):
    """A fresh optimizer: m = v = 0 with scales 0 (the pages initialise the
    scales to zero); the first steps must give the oracle's scales."""
    host = host_tensors([100000, 4096, 7], g_dtype="bf16", p_kind="f16_scaled", p_out="bf16",
                        seed=76, m_v_init="zero")
    assert all(h.scales[1] == 0 and h.scales[2] == 0 for h in host)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 3)
    assert_bitwise(got, ref)


def test_scaled_state_bf16_small_values_overflow_like_the_oracle(torch, orc):
    """bf16 state with moments far below 0.5: the pages' scale is subnormal,
    its reciprocal overflows, and the stored values become +-inf (zeros
    NaN); the library reproduces exactly that."""
    host = host_tensors([5000, 300], g_dtype="bf16", p_kind="bf16_scaled", seed=77,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 1)
    assert_bitwise(got, ref)
    m = (got[0].m.astype(np.uint32) << 16).view(np.float32)
    assert np.isinf(m).sum() > 0


def test_scaled_state_nonfinite_gradient(torch, orc):
    """A NaN gradient makes that tensor's three scales NaN and its stored
    values zeros or NaN; an infinite one makes the param scale infinite.
    Other tensors are unaffected."""
    host = host_tensors([4096, 3000, 700], g_dtype="f32", p_kind="f16_scaled", seed=78,
                        m_v_init="random")
    host[0].g[100] = np.nan
    host[1].g[5] = np.inf
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 1)
    assert_bitwise(got, ref)
    assert np.all(np.isnan(got[0].scales))
    assert np.all(np.isfinite(got[2].scales))


def test_scaled_state_does_not_depend_on_layout(torch, orc):
    """Shared element offsets (peeled heads), unaligned per-stream offsets
    (element path) and chunk sizes give the same bits."""
    sizes = [70001, 4099, 1021, 17]
    host = host_tensors(sizes, g_dtype="bf16", p_kind="f16_scaled", p_out="f16", seed=79,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    roles = ("p", "m", "v", "g", "p_out", "scales")
    results = []
    for offsets, chunk in ((None, 0), ([{r: k % 8 for r in roles} for k in range(4)], 4096),
                           ([{"p": 1, "m": 2, "v": 3, "g": 0, "p_out": 5, "scales": 1}] * 4, 1024)):
        got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 3, desc_kw=dict(chunk_elems=chunk),
                             offsets=offsets)
        assert_bitwise(got, ref, ctx=f"{chunk}")
        results.append(got)
    for r in results[1:]:
        assert_bitwise(r, results[0])


def test_scaled_state_sumsq_and_clip_apply(torch, orc):
    """The gradient reduction reads a scaled-state handle's gradients like
    any other (fp16 gradients here)."""
    host = host_tensors([70001, 333], g_dtype="f16", p_kind="f16_scaled", seed=80)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d = torch.zeros(1, dtype=torch.float64, device="cuda")
    A.adam_grad_sumsq(tl, d)
    torch.cuda.synchronize()
    want = orc.grad_sumsq([h.g for h in host])
    assert abs(float(d.item()) - want) <= 1e-12 * want
    tl.destroy()


# ---------------------------------------------------------------------------
# The maxima pass: approximate params with an error bound, exact recompute of
# the elements that can hold the maximum, and the cases that take the exact
# path for a whole wave or call
# ---------------------------------------------------------------------------

def _f16_scaled(sizes, seed, **kw):
    kw.setdefault("g_dtype", "bf16")
    kw.setdefault("m_v_init", "random")
    return host_tensors(sizes, p_kind="f16_scaled", p_out="f16", seed=seed, **kw)


@pytest.mark.parametrize("mode", [0, 1])
def test_scaled_maxima_with_ties(torch, orc, mode):
    """Many elements at or next to the largest magnitude: a tensor with every
    element equal, one with equal params and gradients one ulp apart, and one
    whose params take three values.  Each of those elements must be
    recomputed exactly; the scales and stored values match the oracle."""
    rng = np.random.default_rng(84)
    host = _f16_scaled([70001, 4096, 3000], 81, g_dtype="f32")
    t = host[0]
    for a in (t.p, t.m, t.v, t.g):
        a[:] = a[17]
    t = host[1]
    t.p[:] = t.p[5]
    t.m[:] = t.m[5]
    t.v[:] = t.v[5]
    base = np.float32(2.5e-3)
    t.g[:] = np.where(rng.random(t.g.size) < 0.5, base, np.nextafter(base, np.float32(1.0)))
    t = host[2]
    t.p[:] = rng.choice(t.p[:3], size=t.p.size)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 3)
    assert_bitwise(got, ref, ctx=f"mode {mode}")


@pytest.mark.parametrize("eps,lr,label", [
    (0.0, 1.6e-3, "eps zero (zero moments give 0/0)"),
    (-1e-8, 1.6e-3, "negative eps (no approximation in the call)"),
    (1e30, 1.6e-3, "large eps"),
    (1e38, 1.6e-3, "eps beyond 2^125 (no approximation in the call)"),
    (1e-8, 1e30, "lr large enough to overflow the update"),
    (1e-8, 0.0, "lr zero"),
    (1e-8, -1e-3, "negative lr"),
])
def test_scaled_maxima_hyperparameter_edges(torch, orc, eps, lr, label):
    """Hyperparameters at the edges of the bound's assumptions (and past
    them), with some elements of zero moments and zero gradient."""
    host = _f16_scaled([70001, 513, 4096], 82)
    for t in host[1:]:
        t.m[:40] = 0
        t.v[:40] = 0
        t.g[:40] = 0
    hl, hr = hp_pair(0.9, 0.95, eps, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, lr, 2)
    assert_bitwise(got, ref, ctx=label)


@pytest.mark.parametrize("mode", [0, 1])
def test_scaled_maxima_subnormal_second_moment(torch, orc, mode):
    """Gradients of ~1e-21 make v_hat subnormal, where the hardware square
    root flushes to zero: the waves holding such elements are recomputed
    exactly (the first tensor throughout, the second at every 97th element)."""
    host = _f16_scaled([70001, 4096], 83, g_dtype="f32", m_v_init="zero", g_std=1e-21)
    t = host[1]
    t.g[:] = np.random.default_rng(85).standard_normal(t.g.size).astype(np.float32) * np.float32(1e-3)
    t.g[::97] = np.float32(3e-21)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
    assert_bitwise(got, ref, ctx=f"mode {mode}")


@pytest.mark.parametrize("mode", [0, 1])
def test_scaled_maxima_negative_subnormal_second_moment(torch, orc, mode):
    """One element of a tensor whose other second moments are normal holds a
    negative stored v that unscales to a subnormal, with zero param, first
    moment and gradient: its v_hat is a negative subnormal, whose exact root
    is NaN (so the tensor's new param scale is NaN) while the hardware root
    flushes it to -0 and the approximate param is 0, far below the cut.  The
    wave must be recomputed exactly."""
    host = _f16_scaled([70001, 4096], 88, g_dtype="f32")
    t = host[1]
    t.scales[2] = np.float32(1e-33)
    t.v[:] = (np.abs(np.random.default_rng(89).standard_normal(t.v.size)) * 1000 + 1).astype(np.float16)
    t.v[77] = np.uint16(0x8001).view(np.float16)  # the smallest negative fp16 subnormal
    t.p[77] = t.m[77] = 0
    t.g[77] = 0
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 1)
    assert np.isnan(ref[1].scales[0])
    assert_bitwise(got, ref, ctx=f"mode {mode}")


@pytest.mark.parametrize("p_kind", ["f16_scaled", "bf16_scaled"])
def test_scaled_maxima_wide_magnitudes(torch, orc, p_kind):
    """Stored params drawn over every finite 16-bit pattern (fp16 subnormals to
    65504; bf16 over all its binades) with large moments: the maxima are
    decided among values of very different sizes, some overflowing."""
    rng = np.random.default_rng(86)
    host = host_tensors([70001, 4096, 1000], p_kind=p_kind, p_out="f16", seed=87, g_dtype="f32",
                        m_v_init="large", g_std=1.0)
    for t in host:
        finite = 0x7C00 if p_kind == "f16_scaled" else 0x7F80
        bits = rng.integers(0, finite, size=t.p.size).astype(np.uint16) | \
            (rng.integers(0, 2, size=t.p.size).astype(np.uint16) << 15)
        t.p[:] = bits.view(t.p.dtype)
    for mode in (0, 1):
        hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
        got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
        assert_bitwise(got, ref, ctx=f"{p_kind} mode {mode}")



# ---------------------------------------------------------------------------
# The capturable scaled-state step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p_kind,g_dtype,p_out,mode", [("f16_scaled", "bf16", "bf16", 1),
                                                       ("bf16_scaled", "f32", "f16", 0)])
def test_scaled_capturable_equals_noncapturable_and_oracle(torch, orc, p_kind, g_dtype, p_out, mode):
    """Device lr (changed every step), grad scale and counter, with the noop
    flag raised on two of six steps: values and scales equal the oracle's
    (which skips those steps), the counter counts the steps that ran, and the
    non-capturable step over the same steps gives the same bits."""
    init = "large" if p_kind == "bf16_scaled" else "random"
    g_std = 1.0 if p_kind == "bf16_scaled" else 1e-3
    host = host_tensors(SIZES, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out, seed=88, m_v_init=init,
                        g_std=g_std)
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_scale = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = [(1e-3, 0), (2e-3, 1), (1.6e-3, 0), (5e-4, 0), (1e-3, 1), (3e-3, 0)]
    ot, st = oracle_tensors(ref), [0]
    for lr, noop in plan:
        d_lr.fill_(lr)
        d_noop.fill_(noop)
        A.adam_step_scaled_capturable(tl, hl, d_lr, d_step, d_scale, d_noop)
        orc.group_step(ot, hr, lr, st, 0.5, noop=noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == st[0] == 4
    got = dev.readback()
    tl.destroy()
    assert_bitwise(got, ref, ctx=f"{p_kind}/{mode}")

    dev2 = DeviceSet(host)
    tl2 = A.adam_tl_build(dev2.tensors, desc_for(host))
    step = A.HostStep(0)
    for lr, noop in plan:
        if not noop:
            A.adam_step_scaled(tl2, hl, lr, step, 0.5)
    torch.cuda.synchronize()
    assert_bitwise(dev2.readback(), got, ctx="non-capturable")
    tl2.destroy()


def test_scaled_capturable_graph_replay(torch, orc):
    """One capturable scaled step recorded in a HIP graph and replayed four
    times, lr changed and the noop flag raised between replays: each
    replay's values and scales follow the oracle."""
    host = host_tensors([70001, 4096, 513], g_dtype="bf16", p_kind="f16_scaled", p_out="f16", seed=89,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr = torch.tensor([1e-3], dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        A.adam_step_scaled_capturable(tl, hl, d_lr, d_step, None, d_noop)
    torch.cuda.synchronize()
    assert int(d_step.item()) == 0
    ref = copies(host)
    ot, st = oracle_tensors(ref), [0]
    for lr, noop in [(1e-3, 0), (2e-3, 1), (5e-4, 0), (1.6e-3, 0)]:
        d_lr.fill_(lr)
        d_noop.fill_(noop)
        graph.replay()
        torch.cuda.synchronize()
        orc.group_step(ot, hr, lr, st, 1.0, noop=noop)
        assert_bitwise(dev.readback(), ref, ctx=f"replay lr {lr} noop {noop}")
    assert int(d_step.item()) == st[0] == 3
    tl.destroy()


# ---------------------------------------------------------------------------
# 16-bit state (p, m, v all bf16 or all fp16) and the fp32 param-out
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p_kind", ["bf16", "f16"])
@pytest.mark.parametrize("g_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("p_out", [None, "f32", "bf16", "f16"])
def test_state16_matches_the_oracle(torch, orc, p_kind, g_dtype, p_out):
    """Every gradient and param-out type with bf16 and fp16 state, three steps
    (L2 for fp16 state, AdamW for bf16), bitwise: p, m, v rounded to the
    state type, the param-out cast from the new stored param."""
    host = host_tensors(SIZES, g_dtype=g_dtype, p_kind=p_kind, p_out=p_out or False, seed=96,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 0 if p_kind == "f16" else 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 3, grad_scale=0.5)
    assert_bitwise(got, ref, ctx=f"{p_kind}/{g_dtype}/{p_out}")


def test_state16_fp16_range_edges(torch, orc):
    """fp16 state next to fp16's limits: params at and near 65504 (the update
    can round them to infinity), subnormal second moments and first moments,
    gradients that make v overflow, and a NaN and an infinite gradient (the
    non-capturable step propagates them)."""
    host = host_tensors([4096, 1000, 33], g_dtype="f32", p_kind="f16", p_out="f32", seed=97,
                        m_v_init="random")
    t = host[0]
    t.p[:8] = np.array([65504.0, -65504.0, 65472.0, 65000.0, 6.1e-5, 6e-8, -6e-8, 0.0], np.float16)
    t.g[:8] = np.array([-1.0, 1.0, -1e3, 300.0, 1e-7, 1e-9, 1e-30, 0.0], np.float32)
    t.m[8:16] = np.float16(6e-8)
    t.v[8:16] = np.float16(6e-8)
    t.g[20], t.g[21] = np.float32(np.nan), np.float32(np.inf)
    host[1].g[:] = np.float32(500.0)  # v' = 0.05 * 500^2 > 65504: infinity
    for mode in (0, 1):
        hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
        got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
        assert_bitwise(got, ref, ctx=f"mode {mode}")


def test_state16_bf16_nonfinite_and_tiny(torch, orc):
    """bf16 state with a NaN and an infinite gradient, subnormal bf16 moments
    and params of very different magnitudes, with an fp16 param-out (which
    overflows for the large ones)."""
    host = host_tensors([4096, 333], g_dtype="bf16", p_kind="bf16", p_out="f16", seed=100,
                        m_v_init="random")
    t = host[0]
    t.g[5], t.g[6] = np.uint16(0x7FC0), np.uint16(0x7F80)  # NaN, +inf
    t.m[100:110] = np.uint16(0x0001)  # smallest subnormal
    t.v[100:110] = np.uint16(0x0001)
    t.p[200:210] = np.array([0x7F00, 0xFF00, 0x4780, 0x0080, 0x8080, 0x3F80, 0x5000, 0x1000, 0x0001, 0x8001],
                            np.uint16)
    for mode in (0, 1):
        hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, mode)
        got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
        assert_bitwise(got, ref, ctx=f"mode {mode}")


@pytest.mark.parametrize("p_kind,p_out", [("bf16", "bf16"), ("f16", "f32")])
def test_state16_capturable_noop_and_graph_replay(torch, orc, p_kind, p_out):
    """The capturable step on 16-bit state: eager calls with device lr and a
    noop step, then the call recorded in a graph and replayed, every result
    against the oracle."""
    host = host_tensors([70001, 4096, 513], g_dtype="bf16", p_kind=p_kind, p_out=p_out, seed=98,
                        m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    ref = copies(host)
    dev = DeviceSet(host)
    tl = A.adam_tl_build(dev.tensors, desc_for(host))
    d_lr = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    ot, st = oracle_tensors(ref), [0]
    for lr, noop in [(1e-3, 0), (2e-3, 1), (1.6e-3, 0)]:
        d_lr.fill_(lr)
        d_noop.fill_(noop)
        A.adam_step_capturable(tl, hl, d_lr, d_step, None, d_noop)
        orc.group_step(ot, hr, lr, st, 1.0, noop=noop)
    torch.cuda.synchronize()
    assert_bitwise(dev.readback(), ref, ctx="eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        A.adam_step_capturable(tl, hl, d_lr, d_step, None, d_noop)
    torch.cuda.synchronize()
    for lr, noop in [(5e-4, 0), (1e-3, 1), (2e-3, 0)]:
        d_lr.fill_(lr)
        d_noop.fill_(noop)
        graph.replay()
        torch.cuda.synchronize()
        orc.group_step(ot, hr, lr, st, 1.0, noop=noop)
        assert_bitwise(dev.readback(), ref, ctx=f"replay {lr} {noop}")
    assert int(d_step.item()) == st[0] == 4
    tl.destroy()


def test_fp32_param_out_is_the_new_param(torch, orc):
    """fp32 params with an fp32 param-out: the copy equals the new param bit
    for bit, and both equal the oracle."""
    host = host_tensors(SIZES, g_dtype="bf16", p_kind="f32", p_out="f32", seed=99, m_v_init="random")
    hl, hr = hp_pair(0.9, 0.95, 1e-8, 0.1, 1)
    got, ref = run_steps(orc, host, hl, hr, 1.6e-3, 2)
    assert_bitwise(got, ref)
    for t in got:
        assert np.array_equal(t.p_out.view(np.uint32), t.p.view(np.uint32))
