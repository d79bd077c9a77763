"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic chunking, the default kernels): the initial state
of sampled elements is copied to the host before the steps run, the oracle
updates those elements one by one, and the GPU's results at the same
positions must match bit for bit.  Samples: whole tensors at the start,
middle and end of each list (or slices of the very large ones) plus random
positions across the flat buffers."""
import gc

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import dev_to_np, torch_mod
from workloads import device_flat, split_views, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()
    return t


@pytest.fixture(autouse=True)
def free_memory():
    yield
    t = torch_mod()
    gc.collect()
    if t.cuda.is_available():
        t.cuda.empty_cache()


def sample_positions(sizes, rng, whole_limit=4_000_000, random_count=1 << 16):
    """Flat positions: the first, middle and last tensor (the last
    `whole_limit` elements of any that is larger), plus random positions."""
    offs = np.concatenate([[0], np.cumsum(sizes)])
    picks = []
    for k in sorted({0, len(sizes) // 2, len(sizes) - 1}):
        lo, hi = offs[k], offs[k + 1]
        picks.append(np.arange(max(lo, hi - whole_limit), hi, dtype=np.int64))
    picks.append(rng.integers(0, offs[-1], size=random_count, dtype=np.int64))
    return np.unique(np.concatenate(picks))


def gather(torch, buf, pos_dev):
    return dev_to_np(buf.index_select(0, pos_dev))


def group_tensors(bufs, sizes, off):
    n = sum(sizes)
    views = {k: split_views(v[off:off + n], sizes) for k, v in bufs.items()}
    return [{k: views[k][i] for k in views} for i in range(len(sizes))]


def out_type(w):
    return ("bf16" if w.p_out is True else w.p_out) or None


def oracle_sample(host, pos, out, rem):
    return oracle.OracleTensor(p=host["p"].copy(), m=host["m"].copy(), v=host["v"].copy(),
                               g=host["g"].copy(),
                               p_out=None if not out else np.zeros(len(pos), np.float16 if out == "f16"
                                                                   else np.uint16),
                               rem=host["rem"].copy() if rem else None)


def compare(got, ref, roles):
    for r in roles:
        a, b = got[r], getattr(ref, r)
        if a.dtype == np.float32:
            same = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
        elif a.dtype == np.float16:
            same = (a.view(np.uint16) == b.view(np.uint16)) | (np.isnan(a) & np.isnan(b))
        else:
            same = a == b
        assert same.all(), f"{r}: {int((~same).sum())} of {a.size} sampled elements differ"


def run_sampled(torch, wname, steps, *, capturable=False, noop_every=0, seed=0,
                whole_limit=4_000_000, two_buffer=False):
    """With `two_buffer`, each group's handle also gets a second set of p, m,
    v (and rem), filled with 0x7B bytes; at the end the sampled state must
    be the oracle's in set (steps taken & 1) and its state one step earlier
    in the other set."""
    w = workloads()[wname]
    rng = np.random.default_rng(seed)
    groups = [(w.sizes, w.weight_decay)] + list(w.extra_groups)
    bufs = device_flat(w.numel, g_dtype=w.g_dtype, p_kind=w.p_kind, p_out=w.p_out, seed=w.seed,
                       g_multiplier=w.grad_multiplier)
    torch.cuda.synchronize()
    rem = w.p_kind == "bf16_rem"
    roles = [r for r in ("p", "rem", "m", "v", "g") if r in bufs]
    out_roles = ["p", "m", "v"] + (["rem"] if rem else []) + (["p_out"] if w.p_out else [])
    state_roles = [r for r in ("p", "rem", "m", "v") if r in bufs]
    alt = {}
    if two_buffer:
        for r in state_roles:
            alt[r] = torch.empty_like(bufs[r])
            alt[r].view(torch.uint8).fill_(0x7B)
    handles, samples = [], []
    off = 0
    for sizes, wd in groups:
        n = sum(sizes)
        pos = sample_positions(sizes, rng, whole_limit) + off
        pos_dev = torch.from_numpy(pos).to("cuda")
        host = {r: gather(torch, bufs[r], pos_dev) for r in roles}
        alts = group_tensors(alt, sizes, off) if two_buffer else None
        tl = A.adam_tl_build(group_tensors(bufs, sizes, off),
                             A.make_desc(g=w.g_dtype, p=w.p_kind, p_out=out_type(w)), alternates=alts)
        hp = A.AdamHParams(w.beta1, w.beta2, w.eps, wd, w.mode, 1)
        hr = oracle.HParams(w.beta1, w.beta2, w.eps, wd, w.mode, 1)
        handles.append(dict(tl=tl, hp=hp, hr=hr, step=A.HostStep(0),
                            d_step=torch.zeros(1, dtype=torch.int32, device="cuda"), ref_step=[0]))
        samples.append(dict(pos=pos, pos_dev=pos_dev, ref=oracle_sample(host, pos, out_type(w), rem)))
        off += n
    d_scale = torch.tensor([w.grad_scale], dtype=torch.float32, device="cuda")
    d_lr = torch.tensor([w.lr], dtype=torch.float32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    inf_pos = int(samples[0]["pos"][len(samples[0]["pos"]) // 3])
    o = oracle.default()
    for k in range(1, steps + 1):
        skip = noop_every and k % noop_every == 0
        if skip:
            saved = float(bufs["g"][inf_pos].item())
            bufs["g"][inf_pos] = float("inf")
            d_noop.fill_(1)
            if k == noop_every:  # full-buffer check once
                before = {r: bufs[r].clone() for r in out_roles}
        for h in handles:
            if capturable and rem:
                A.adam_step_remainders_capturable(h["tl"], h["hp"], d_lr, h["d_step"], d_scale, d_noop)
            elif capturable:
                A.adam_step_capturable(h["tl"], h["hp"], d_lr, h["d_step"], d_scale, d_noop)
            elif rem:
                A.adam_step_remainders(h["tl"], h["hp"], w.lr, h["step"], 1.0, d_scale)
            else:
                A.adam_step(h["tl"], h["hp"], w.lr, h["step"], 1.0, d_scale)
        if skip:
            torch.cuda.synchronize()
            if k == noop_every:
                for r in out_roles:
                    assert torch.equal(before[r], bufs[r]), f"noop step changed {r}"
                del before
            bufs["g"][inf_pos] = saved
            d_noop.fill_(0)
        for h, smp in zip(handles, samples):
            if two_buffer and not skip:
                smp["prev"] = {r: getattr(smp["ref"], r).copy() for r in state_roles}
            o.group_step([smp["ref"]], h["hr"], w.lr, h["ref_step"], w.grad_scale,
                         noop=(1 if skip else 0) if capturable else None)
    torch.cuda.synchronize()
    for h, smp in zip(handles, samples):
        cur = alt if two_buffer and h["ref_step"][0] & 1 else bufs
        got = {r: gather(torch, cur[r] if r in state_roles else bufs[r], smp["pos_dev"]) for r in out_roles}
        compare(got, smp["ref"], out_roles)
        if two_buffer:
            other = bufs if cur is alt else alt
            before = oracle.OracleTensor(**{r: smp["prev"].get(r) for r in ("p", "m", "v", "rem")},
                                         g=None, p_out=None)
            compare({r: gather(torch, other[r], smp["pos_dev"]) for r in state_roles}, before, state_roles)
        want_steps = steps - (steps // noop_every if noop_every else 0)
        assert h["ref_step"][0] == want_steps
        if capturable:
            assert int(h["d_step"].item()) == want_steps
        else:
            assert h["step"].value == want_steps
        h["tl"].destroy()
    return bufs


def test_bench201_ten_steps(torch):
    """201 fp32 tensors of 20,971,520 elements, AdamW, ten non-capturable
    steps (the benchmark's workload and launch)."""
    run_sampled(torch, "bench201", 10, seed=1)


def test_bench201_capturable_ten_steps(torch):
    run_sampled(torch, "bench201", 10, capturable=True, seed=2)


def test_shard30b_two_groups_ten_steps(torch):
    """30B-class shard: decay group (337 tensors) and no-decay norms (48),
    bf16 loss-scaled grads unscaled by a device grad scale of 2^-16."""
    run_sampled(torch, "shard30b", 10, seed=3)


def test_zero_shard_capturable_with_noop_every_fifth_step(torch):
    """1e9-element ZeRO shard in 2048 buckets, bf16 grads and bf16 p_out,
    capturable with a device step; steps 5, 10, 15, 20 carry an infinite
    gradient and the noop flag, and must leave every buffer untouched."""
    run_sampled(torch, "zero1e9", 20, capturable=True, noop_every=5, seed=4)


def test_remainders_hundred_steps_with_empty_group(torch):
    """5e8 elements as bf16 params + int16 remainders in ragged tensors,
    100 steps; an empty group's counter advances every step."""
    empty = A.adam_tl_build([], A.make_desc(p="bf16_rem", g="bf16"), stream=0)
    empty_step = A.HostStep(0)
    bufs = run_sampled(torch, "rem5e8", 100, seed=5, whole_limit=1_000_000)
    for _ in range(100):
        A.adam_step_remainders(empty, A.AdamHParams(), 1e-3, empty_step)
    assert empty_step.value == 100
    del bufs


def test_zero_shard_fp16_capturable_with_noop(torch):
    """The ZeRO shard with fp16 gradients and an fp16 param-sync copy,
    capturable, noop on every 5th step."""
    run_sampled(torch, "zero1e9_f16", 10, capturable=True, noop_every=5, seed=8)


@pytest.mark.parametrize("capturable,passes", [(False, 1), (True, 1), (False, 2), (True, 2)])
def test_scaled_state_zero_shard(torch, capturable, passes):
    """1e9 elements of scaled fp16 p, m, v in 2048 buckets, bf16 gradients,
    bf16 param-sync copy, in one pass and in two, five steps from a fresh state (capturable: six
    calls from device scalars, the fourth a noop).  The new scales of a
    tensor depend on all of it, so the samples are whole tensors (first,
    middle, last and five random buckets): their initial state goes to the
    host, the oracle steps them, and values, scales and p_out must match."""
    w = workloads()["scaled1e9"]
    from workloads import scaled_p_scale

    bufs = device_flat(w.numel, g_dtype=w.g_dtype, p_kind=w.p_kind, p_out=w.p_out, seed=w.seed)
    sizes = w.sizes
    offs = np.concatenate([[0], np.cumsum(sizes)])
    scales = torch.zeros((len(sizes), 3), dtype=torch.float32, device="cuda")
    scales[:, 0] = scaled_p_scale(w.p_kind)
    tensors = group_tensors(bufs, sizes, 0)
    for i, t in enumerate(tensors):
        t["scales"] = scales[i]
    rng = np.random.default_rng(9)
    picks = sorted({0, len(sizes) // 2, len(sizes) - 1, *rng.integers(0, len(sizes), 5).tolist()})
    torch.cuda.synchronize()
    refs = []
    for k in picks:
        lo, hi = int(offs[k]), int(offs[k + 1])
        host = {r: dev_to_np(bufs[r][lo:hi]) for r in ("p", "m", "v", "g")}
        refs.append(oracle.OracleTensor(host["p"], host["m"], host["v"], host["g"],
                                        np.zeros(hi - lo, np.uint16), None,
                                        dev_to_np(scales[k]).astype(np.float32)))
    tl = A.adam_tl_build(tensors, A.make_desc(g=w.g_dtype, p=w.p_kind, p_out=out_type(w), scaled_passes=passes))
    assert tl.info()["scaled_passes"] == passes
    hp = A.AdamHParams(w.beta1, w.beta2, w.eps, w.weight_decay, w.mode, 1)
    hr = oracle.HParams(w.beta1, w.beta2, w.eps, w.weight_decay, w.mode, 1)
    step, ref_step = A.HostStep(0), [0]
    if capturable:
        d_lr = torch.tensor([w.lr], dtype=torch.float32, device="cuda")
        d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
        d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
        for k in range(6):
            d_noop.fill_(1 if k == 3 else 0)
            A.adam_step_scaled_capturable(tl, hp, d_lr, d_step, None, d_noop)
            oracle.default().group_step(refs, hr, w.lr, ref_step, 1.0, noop=1 if k == 3 else 0)
        torch.cuda.synchronize()
        assert int(d_step.item()) == ref_step[0] == 5
    else:
        for _ in range(5):
            A.adam_step_scaled(tl, hp, w.lr, step)
            oracle.default().group_step(refs, hr, w.lr, ref_step, 1.0)
        torch.cuda.synchronize()
        assert step.value == ref_step[0] == 5
    for k, ref in zip(picks, refs):
        lo, hi = int(offs[k]), int(offs[k + 1])
        got = {r: dev_to_np(bufs[r][lo:hi]) for r in ("p", "m", "v", "p_out")}
        got["scales"] = dev_to_np(scales[k])
        compare(got, ref, ("p", "m", "v", "p_out", "scales"))
    tl.destroy()


def test_state16_shard_capturable_with_noop(torch):
    """The ZeRO shard with bf16 optimizer state (p, m, v), bf16 gradients and
    a bf16 param-sync copy through the capturable step, noop on every 4th
    step."""
    run_sampled(torch, "state16_1e9", 12, capturable=True, noop_every=4, seed=11)


def test_remainders_capturable_with_noop(torch):
    """The remainder workload through the capturable remainder step, noop on
    every 4th step."""
    run_sampled(torch, "rem5e8", 12, capturable=True, noop_every=4, seed=10, whole_limit=1_000_000)


def test_bench201_two_buffer_state_ten_steps(torch):
    """The benchmark's list with a second buffer set (its two-buffer
    measurement): ten host steps, then the state in set 0 and the state one
    step earlier in set 1."""
    run_sampled(torch, "bench201", 10, seed=12, two_buffer=True)


def test_zero_shard_two_buffer_capturable_with_noop(torch):
    """The ZeRO shard with a second buffer set through the capturable step,
    noop on every 4th step: the side follows the device counter."""
    run_sampled(torch, "zero1e9", 11, capturable=True, noop_every=4, seed=13, two_buffer=True)


def test_remainders_two_buffer_state(torch):
    run_sampled(torch, "rem5e8", 7, seed=14, whole_limit=1_000_000, two_buffer=True)


def test_single_tensor_beyond_2_pow_31_elements(torch):
    """One tensor of 2^31 + 5 elements (fp32 p/m/v, bf16 g): positions past
    2^31 are updated like the rest."""
    n = (1 << 31) + 5
    bufs = device_flat(n, g_dtype="bf16", p_kind="f32", p_out=False, seed=6)
    rng = np.random.default_rng(6)
    pos = np.unique(np.concatenate([np.arange(n - 4096, n), rng.integers(0, n, 4096)]))
    pos_dev = torch.from_numpy(pos).to("cuda")
    host = {r: gather(torch, bufs[r], pos_dev) for r in ("p", "m", "v", "g")}
    tl = A.adam_tl_build([dict(p=bufs["p"], m=bufs["m"], v=bufs["v"], g=bufs["g"])],
                         A.make_desc(g="bf16"))
    hp = A.AdamHParams(0.9, 0.95, 1e-8, 0.1, 1, 1)
    step = A.HostStep(0)
    for _ in range(2):
        A.adam_step(tl, hp, 1.6e-3, step)
    torch.cuda.synchronize()
    ref = oracle_sample(host, pos, False, False)
    st = [0]
    for _ in range(2):
        oracle.default().group_step([ref], oracle.HParams(0.9, 0.95, 1e-8, 0.1, 1, 1), 1.6e-3, st, 1.0)
    compare({r: gather(torch, bufs[r], pos_dev) for r in ("p", "m", "v")}, ref, ("p", "m", "v"))
    tl.destroy()
