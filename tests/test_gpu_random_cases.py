"""Seeded random GPU parity cases: each case draws a dtype set (fp32 or 16-bit
state, remainders, scaled state; fp32 / bf16 / fp16 gradients; no, fp32,
bf16 or fp16 param-out as the storage allows), tensor
sizes (empty, tiny, ragged, several work items), a layout (aligned, one
shared element offset per tensor, or independent offsets per stream),
hyperparameters (L2 or AdamW, bias correction on or off, betas near 1 or
not, eps, weight decay, lr, grad scale on the host or the device), a chunk
size and a number of steps, then runs the library (capturable where the
storage allows it and the case says so, with the noop flag raised on random
steps) and the oracle from the same inputs and compares every output bit
for bit (NaN as NaN) and the step counter.  A third of the cases whose
storage allows it (drawn from a separate seed, so the other draws stay
fixed) give the state a second buffer set; the result is then read from set
(steps taken & 1)."""
import os

import numpy as np
import pytest

import adamw_optimizer_step_tensor_amd as A
import oracle
from gpu_helpers import DeviceSet, assert_bitwise, copies, desc_for, oracle_tensors, torch_mod
from workloads import host_tensors

pytestmark = pytest.mark.gpu

# ADAM_RANDOM_CASES widens the sweep (case k is always drawn from seed 1000 + k)
CASES = int(os.environ.get("ADAM_RANDOM_CASES", "96"))

STORAGE = [  # (p_kind, allowed gradient types, allowed param-out)
    ("f32", ("f32", "bf16", "f16"), (None, "bf16", "f16", "f32")),
    ("bf16", ("f32", "bf16", "f16"), (None, "bf16", "f16", "f32")),
    ("f16", ("f32", "bf16", "f16"), (None, "bf16", "f16", "f32")),
    ("bf16_rem", ("f32", "bf16", "f16"), (None, "bf16")),
    ("f16_scaled", ("f32", "bf16", "f16"), (None, "bf16", "f16")),
    ("bf16_scaled", ("f32", "bf16", "f16"), (None, "bf16", "f16")),
]
SPECIAL_SIZES = [0, 1, 2, 3, 4, 5, 7, 63, 64, 65, 127, 511, 512, 513, 1023, 1024, 4095, 4097]


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


def draw_case(k):
    rng = np.random.default_rng(1000 + k)
    p_kind, gs, outs = STORAGE[int(rng.integers(len(STORAGE)))]
    g_dtype = gs[int(rng.integers(len(gs)))]
    p_out = outs[int(rng.integers(len(outs)))]
    n = int(rng.integers(1, 6))
    sizes = [int(rng.choice(SPECIAL_SIZES)) if rng.random() < 0.5 else int(rng.integers(1, 40000))
             for _ in range(n)]
    layout = ["aligned", "shared", "random"][int(rng.integers(3))]
    mode = int(rng.integers(2))
    bias_correction = int(rng.random() < 0.8)
    beta1 = float(rng.choice([0.0, 0.5, 0.9, 0.99]))
    beta2 = float(rng.choice([0.9, 0.95, 0.999, 0.9999]))
    eps = float(rng.choice([1e-8, 1e-6, 1e-12, 1e-3]))
    wd = float(rng.choice([0.0, 0.01, 0.1]))
    lr = float(rng.choice([1e-3, 1.6e-3, 3e-2]))
    grad_scale = float(rng.choice([1.0, 0.5, 2.0 ** -10]))
    device_scale = bool(rng.random() < 0.5)
    chunk = int(rng.choice([0, 1024, 4096, 65536]))
    steps = int(rng.integers(1, 5))
    capturable = bool(rng.random() < 0.4)
    noops = [int(rng.random() < 0.3) for _ in range(steps)] if capturable else [0] * steps
    two_buffer = not p_kind.endswith("_scaled") and np.random.default_rng(500000 + k).random() < 1 / 3
    return dict(p_kind=p_kind, g_dtype=g_dtype, p_out=p_out, sizes=sizes, layout=layout, mode=mode,
                bias_correction=bias_correction, beta1=beta1, beta2=beta2, eps=eps, wd=wd, lr=lr,
                grad_scale=grad_scale, device_scale=device_scale, chunk=chunk, steps=steps,
                capturable=capturable, noops=noops, seed=2000 + k, rng=rng, two_buffer=two_buffer)


@pytest.mark.parametrize("k", range(CASES))
def test_random_case(torch, orc, k):
    c = draw_case(k)
    rng = c.pop("rng")
    scaled = c["p_kind"].endswith("_scaled")
    init = "large" if c["p_kind"] == "bf16_scaled" else "random"
    host = host_tensors(c["sizes"], g_dtype=c["g_dtype"], p_kind=c["p_kind"], p_out=c["p_out"] or False,
                        seed=c["seed"], m_v_init=init, g_std=1.0 if c["p_kind"] == "bf16_scaled" else 1e-3)
    roles = ("p", "rem", "m", "v", "g", "p_out", "scales")
    if c["layout"] == "aligned":
        offsets = None
    elif c["layout"] == "shared":
        offsets = []
        for _ in c["sizes"]:
            o = int(rng.integers(0, 70))
            offsets.append({r: o for r in roles})
    else:
        offsets = [{r: int(rng.integers(0, 9)) for r in roles} for _ in c["sizes"]]
    ref = copies(host)
    dev = DeviceSet(host, offsets)
    alt = None
    if c["two_buffer"]:
        second = copies(host)  # the second set starts as values no step produces
        for h in second:
            for r in ("p", "m", "v", "rem"):
                a = getattr(h, r)
                if a is not None and a.size:
                    a.view(np.uint8)[...] = 0x7B
        alt = DeviceSet(second, offsets)
        alts = [{r: (d.get(r) if h.p.size else None) for r in ("p", "m", "v", "rem")}
                for d, h in zip(alt.tensors, host)]
        tl = A.adam_tl_build(dev.tensors, desc_for(host, chunk_elems=c["chunk"]), alternates=alts)
    else:
        tl = A.adam_tl_build(dev.tensors, desc_for(host, chunk_elems=c["chunk"]))
    hp = A.AdamHParams(c["beta1"], c["beta2"], c["eps"], c["wd"], c["mode"], c["bias_correction"])
    hr = oracle.HParams(c["beta1"], c["beta2"], c["eps"], c["wd"], c["mode"], c["bias_correction"])
    d_scale = torch.tensor([c["grad_scale"]], dtype=torch.float32, device="cuda")
    ot = oracle_tensors(ref)
    ref_step = [0]
    if c["capturable"]:
        d_lr = torch.tensor([c["lr"]], dtype=torch.float32, device="cuda")
        d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
        d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
        fn = {"bf16_rem": A.adam_step_remainders_capturable, "f16_scaled": A.adam_step_scaled_capturable,
              "bf16_scaled": A.adam_step_scaled_capturable}.get(c["p_kind"], A.adam_step_capturable)
        for noop in c["noops"]:
            d_noop.fill_(noop)
            fn(tl, hp, d_lr, d_step, d_scale, d_noop)
            orc.group_step(ot, hr, c["lr"], ref_step, c["grad_scale"], noop=noop)
        torch.cuda.synchronize()
        assert int(d_step.item()) == ref_step[0] == c["steps"] - sum(c["noops"])
    else:
        fn = {"bf16_rem": A.adam_step_remainders, "f16_scaled": A.adam_step_scaled,
              "bf16_scaled": A.adam_step_scaled}.get(c["p_kind"], A.adam_step)
        step = A.HostStep(0)
        for _ in range(c["steps"]):
            if c["device_scale"]:
                fn(tl, hp, c["lr"], step, 123.0, d_scale)
            else:
                fn(tl, hp, c["lr"], step, c["grad_scale"])
            orc.group_step(ot, hr, c["lr"], ref_step, c["grad_scale"])
        torch.cuda.synchronize()
        assert step.value == ref_step[0] == c["steps"]
    got = dev.readback()
    if alt is not None and ref_step[0] & 1:  # the state is in the second set
        second = alt.readback()
        for gt, sd in zip(got, second):
            gt.p, gt.m, gt.v, gt.rem = sd.p, sd.m, sd.v, sd.rem
    tl.destroy()
    ctx = {k2: v for k2, v in c.items() if k2 != "sizes"} | {"sizes": c["sizes"]}
    assert_bitwise(got, ref, ctx=str(ctx))
    if scaled:
        for t in got:
            assert t.scales is not None
