"""Seeded synthetic inputs for the fused Adam / AdamW step.

This module only draws numbers and describes shapes; it holds none of the
update's arithmetic, so the oracle and the HIP path can both be fed from it.
Shapes and value distributions follow the pages' workloads:

* the benchmark script in TransformerEngine issue "[Performance] FusedAdam
  capturable kernel is ~1.9x slower than regular Adam on GB300" (201 fp32
  tensors of 320*65536 elements, p ~ N(0,1), g ~ N(0,1)*1e-3, lr 1.6e-3,
  betas (0.9, 0.95), eps 1e-8, weight decay 0.1, AdamW);
* a ragged single-GPU shard of a 30B-class transformer (per-layer matrices,
  RMSNorm vectors and an embedding), standing in for the Nemotron training
  run that issue reports on, which is not available here;
* a ZeRO-style local shard cut into buckets (apex distributed_fused_adam.py,
  bucket sizes rounded to the 128-byte alignment of the grad-sync dtype);
* bf16 params with int16 remainders;
* per-tensor scaled 16-bit optimizer state (apex distributed_fused_adam.py,
  ``with_scaled_states``) on the ZeRO shard's buckets.

Host arrays are numpy (bf16 as raw uint16 bits).  Large inputs are drawn on
the GPU with torch's generator (see ``device_*`` helpers) so no 100 GB host
copy is needed; tests that compare such inputs against the oracle copy the
sampled elements' initial values to the host before the step runs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    sizes: Tuple[int, ...]                 # elements per tensor (group 0)
    g_dtype: str                           # "f32", "bf16" or "f16"
    p_kind: str                            # "f32", "bf16" / "f16" (16-bit p, m, v), "bf16_rem",
                                           # "bf16_scaled" or "f16_scaled"
    p_out: object                          # False, True / "bf16", "f16" or "f32": param-out copy
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    mode: int                              # 0 = L2, 1 = AdamW
    grad_scale: float = 1.0
    grad_multiplier: float = 1.0           # loss scale folded into the grads
    seed: int = 0
    extra_groups: Tuple[Tuple[Tuple[int, ...], float], ...] = ()  # (sizes, wd)
    scaled_passes: int = 0                 # scaled state: 1 = one pass, else two

    @property
    def numel(self) -> int:
        return sum(self.sizes) + sum(sum(s) for s, _ in self.extra_groups)

    @property
    def bytes_per_elem(self) -> int:
        """Algorithmic HBM bytes per element: every state word is read once and
        written once; the gradient is read once."""
        state16 = self.p_kind.endswith("_scaled") or self.p_kind in ("bf16", "f16")
        p = 2 if state16 else 4  # fp32 p, bf16 p + int16 rem, or a 16-bit p
        mv = 2 if state16 else 4
        g = 4 if self.g_dtype == "f32" else 2
        out = {None: 0, "f32": 4}.get(_out_type(self.p_out), 2)
        read = p + 2 * mv + g
        write = p + 2 * mv + out
        return read + write


TINY_SIZES = (4096, 1000, 7)

TRANSFORMER_LAYERS = 48
HIDDEN = 4096
KV_DIM = 1024
FFN = 14336
VOCAB = 131072


def transformer_shard_sizes() -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """(decay group sizes, no-decay group sizes) of the 30B-class shard: per
    layer q and o (4096x4096), k and v (4096x1024), two 4096x14336 MLP inputs
    and one 14336x4096 MLP output, and one 4096 RMSNorm vector; plus a
    131072x4096 embedding in the decay group."""
    decay: List[int] = []
    no_decay: List[int] = []
    for _ in range(TRANSFORMER_LAYERS):
        decay += [HIDDEN * HIDDEN, HIDDEN * KV_DIM, HIDDEN * KV_DIM, HIDDEN * HIDDEN,
                  HIDDEN * FFN, HIDDEN * FFN, FFN * HIDDEN]
        no_decay.append(HIDDEN)
    decay.append(VOCAB * HIDDEN)
    return tuple(decay), tuple(no_decay)


def zero_bucket_sizes(total: int = 1_000_000_000, count: int = 2048,
                      lo: int = 65536, hi: int = 2_097_152, align: int = 64,
                      seed: int = 4) -> Tuple[int, ...]:
    """Bucket sizes of a ZeRO local shard: ``count`` sizes drawn log-uniform in
    [lo, hi], scaled (and clamped to the range) until they sum to about
    ``total``, rounded to multiples of ``align`` (64 bf16 elements = 128
    bytes), then nudged one ``align`` at a time, within the range, until the
    sum is exactly ``total``."""
    assert total % align == 0 and lo % align == 0 and hi % align == 0
    assert lo * count <= total <= hi * count
    rng = np.random.default_rng(seed)
    raw = np.exp(rng.uniform(math.log(lo), math.log(hi), size=count))
    f = total / raw.sum()
    for _ in range(100):
        cur = np.clip(raw * f, lo, hi)
        f *= total / cur.sum()
    units = np.clip(np.round(np.clip(raw * f, lo, hi) / align), lo // align, hi // align).astype(np.int64)
    diff = total // align - int(units.sum())
    order = rng.permutation(count)
    i = 0
    while diff != 0:
        k = order[i % count]
        if diff > 0 and units[k] < hi // align:
            units[k] += 1
            diff -= 1
        elif diff < 0 and units[k] > lo // align:
            units[k] -= 1
            diff += 1
        i += 1
    sizes = units * align
    assert int(sizes.sum()) == total and sizes.min() >= lo and sizes.max() <= hi
    return tuple(int(s) for s in sizes)


def ragged_sizes(total: int, count: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    """Ragged tensor sizes (any residue mod 4), log-uniform in [lo, hi],
    scaled to sum to ``total``; the largest tensor absorbs the rounding."""
    rng = np.random.default_rng(seed)
    raw = np.exp(rng.uniform(math.log(lo), math.log(hi), size=count))
    raw *= total / raw.sum()
    sizes = np.maximum(np.floor(raw), 1).astype(np.int64)
    sizes += rng.integers(0, 4, size=count)  # ragged tails
    big = int(np.argmax(sizes))
    sizes[big] += total - int(sizes.sum())
    assert int(sizes.sum()) == total and sizes.min() > 0
    return tuple(int(s) for s in sizes)


def workloads() -> dict:
    decay, no_decay = transformer_shard_sizes()
    return {
        "tiny": Workload("tiny", TINY_SIZES, "f32", "f32", False,
                         lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                         weight_decay=0.01, mode=1, seed=1),
        "bench201": Workload("bench201", (320 * 65536,) * 201, "f32", "f32", False,
                             lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                             weight_decay=0.1, mode=1, seed=2),
        "shard30b": Workload("shard30b", decay, "bf16", "f32", False,
                             lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                             weight_decay=0.1, mode=1, grad_scale=2.0 ** -16,
                             grad_multiplier=65536.0, seed=3,
                             extra_groups=((no_decay, 0.0),)),
        "zero1e9": Workload("zero1e9", zero_bucket_sizes(), "bf16", "f32", True,
                            lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                            weight_decay=0.1, mode=1, seed=4),
        "rem5e8": Workload("rem5e8", ragged_sizes(500_000_000, 300, 1, 8_000_000, seed=5),
                           "bf16", "bf16_rem", False,
                           lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                           weight_decay=0.1, mode=1, seed=5),
        # the ZeRO shard with fp16 gradients and an fp16 param-sync copy
        "zero1e9_f16": Workload("zero1e9_f16", zero_bucket_sizes(), "f16", "f32", "f16",
                                lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                                weight_decay=0.1, mode=1, seed=6),
        # the ZeRO shard with scaled fp16 p, m, v, bf16 gradients and a bf16
        # param-sync copy: 16 B/elem
        "scaled1e9": Workload("scaled1e9", zero_bucket_sizes(), "bf16", "f16_scaled", "bf16",
                              lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                              weight_decay=0.1, mode=1, seed=7),
        # the same, stepped in one pass (each input read once)
        "scaled1e9_one": Workload("scaled1e9_one", zero_bucket_sizes(), "bf16", "f16_scaled", "bf16",
                                  lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                                  weight_decay=0.1, mode=1, seed=7, scaled_passes=1),
        # the ZeRO shard with the optimizer state in bf16 (p, m, v), bf16
        # gradients and a bf16 param-sync copy (apex's gradient and param-sync
        # dtypes default to the state dtype): 16 B/elem
        "state16_1e9": Workload("state16_1e9", zero_bucket_sizes(), "bf16", "bf16", "bf16",
                                lr=1.6e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                                weight_decay=0.1, mode=1, seed=8),
    }


# ---------------------------------------------------------------------------
# Host (numpy) inputs
# ---------------------------------------------------------------------------


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits with torch's CPU cast (a library conversion: the
    input generator does not use either side's rounding code)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class HostTensor:
    p: np.ndarray                        # float32, bf16 bits (uint16) or float16 (scaled)
    m: np.ndarray                        # float32, or p's 16-bit type (scaled)
    v: np.ndarray                        # float32, or p's 16-bit type (scaled)
    g: np.ndarray                        # float32, bf16 bits (uint16) or float16
    p_out: Optional[np.ndarray] = None   # bf16 bits (uint16) or float16
    rem: Optional[np.ndarray] = None     # int16
    scales: Optional[np.ndarray] = None  # float32[3] (scaled state)

    def copy(self) -> "HostTensor":
        c = lambda a: None if a is None else a.copy()
        return HostTensor(c(self.p), c(self.m), c(self.v), c(self.g), c(self.p_out),
                          c(self.rem), c(self.scales))


# Scaled-state inputs: stored = T(x * 2^k), scale = 2^-k, with k per buffer
# chosen so that the drawn magnitudes sit well inside fp16's range (bf16
# shares fp32's range and takes k = 0).  Any (stored, scale) pair is a valid
# state; these are not the method's own scaling.
_F16_SHIFT = {"p": 12, "m": 22, "v": 32}


def _to_state(x: np.ndarray, state: str, role: str):
    k = _F16_SHIFT[role] if state == "f16" else 0
    y = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
    stored = y.astype(np.float16) if state == "f16" else _to_bf16_bits(y)
    return stored, np.float32(2.0 ** -k)


def _out_type(p_out) -> Optional[str]:
    """p_out option: False/None (absent), True or "bf16", "f16", or "f32"."""
    if p_out is None or p_out is False:
        return None
    return "bf16" if p_out is True else p_out


def host_tensors(sizes: Sequence[int], *, g_dtype: str = "f32", p_kind: str = "f32",
                 p_out=False, seed: int = 0, g_std: float = 1e-3,
                 g_multiplier: float = 1.0, m_v_init: str = "zero") -> List[HostTensor]:
    """p ~ N(0,1), g ~ N(0,1)*g_std*g_multiplier (g_dtype "f32", "bf16" or
    "f16", cast by library conversions).  m = v = 0 by default;
    ``m_v_init="random"`` draws m ~ N(0,1)*1e-3 and v ~ |N(0,1)|*1e-6 (a
    state part-way through training); ``"large"`` draws m ~ N(0,1)*4 and
    v ~ |N(0,1)|*4 + 1.  Remainder params (p_kind "bf16_rem"): bf16 p drawn as
    the cast of N(0,1) and the int16 remainder uniform over all 65536 values,
    so every (bf16, remainder) pair is a valid master weight.  16-bit state
    (p_kind "bf16" / "f16"): p, m, v are the casts of the fp32 draws.  Scaled state
    (p_kind "bf16_scaled" / "f16_scaled"): p, m, v stored as T(x * 2^k) with
    scale 2^-k (zero moments get scale 0, as a fresh optimizer has them).
    p_out: False, True / "bf16", "f16", or "f32"."""
    rng = np.random.default_rng(seed)
    out_type = _out_type(p_out)
    out = []
    for n in sizes:
        p32 = rng.standard_normal(n, dtype=np.float32)
        g32 = (rng.standard_normal(n, dtype=np.float32) * np.float32(g_std)
               * np.float32(g_multiplier)).astype(np.float32)
        if m_v_init == "zero":
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
        elif m_v_init == "large":
            m = (rng.standard_normal(n, dtype=np.float32) * np.float32(4.0)).astype(np.float32)
            v = (np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(4.0)
                 + np.float32(1.0)).astype(np.float32)
        else:
            m = (rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)).astype(np.float32)
            v = (np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(1e-6)).astype(np.float32)
        g = {"f32": lambda x: x, "bf16": _to_bf16_bits,
             "f16": lambda x: x.astype(np.float16)}[g_dtype](g32)
        rem = scales = None
        if p_kind == "f32":
            p = p32
        elif p_kind in ("bf16", "f16"):  # 16-bit state: p, m, v of one 16-bit type
            cast = (lambda x: x.astype(np.float16)) if p_kind == "f16" else _to_bf16_bits
            p, m, v = cast(p32), cast(m), cast(v)
        elif p_kind == "bf16_rem":
            p = _to_bf16_bits(p32)
            rem = rng.integers(-32768, 32768, size=n, dtype=np.int64).astype(np.int16)
        else:
            state = {"bf16_scaled": "bf16", "f16_scaled": "f16"}[p_kind]
            p, sp = _to_state(p32, state, "p")
            m, sm = _to_state(m, state, "m")
            v, sv = _to_state(v, state, "v")
            if m_v_init == "zero":
                sm = sv = np.float32(0.0)
            scales = np.array([sp, sm, sv], np.float32)
        po = None if out_type is None else np.zeros(n, {"f16": np.float16, "bf16": np.uint16,
                                                         "f32": np.float32}[out_type])
        out.append(HostTensor(p, m, v, g, po, rem, scales))
    return out


# ---------------------------------------------------------------------------
# Device (torch) inputs for full-size workloads
# ---------------------------------------------------------------------------


def device_flat(total: int, *, g_dtype: str, p_kind: str, p_out, seed: int,
                device="cuda", g_std: float = 1e-3, g_multiplier: float = 1.0,
                chunk: int = 1 << 28):
    """Flat device buffers for ``total`` elements, drawn with torch's CUDA
    generator in chunks: p ~ N(0,1), g ~ N(0,1)*g_std*g_multiplier, m = v = 0.
    Returns a dict of torch tensors (bf16 kept as torch.bfloat16, fp16 as
    torch.float16; remainders as torch.int16).  Scaled state stores p as
    T(p * 2^k) (k from the scaled-state recipe); the caller keeps the scales
    ([2^-k, 0, 0] per tensor, see ``scaled_p_scale``)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    bufs = {}
    scaled = p_kind in ("bf16_scaled", "f16_scaled")
    if p_kind == "f32":
        bufs["p"] = torch.empty(total, dtype=torch.float32, device=device)
    elif p_kind == "bf16_rem":
        bufs["p"] = torch.empty(total, dtype=torch.bfloat16, device=device)
        bufs["rem"] = torch.empty(total, dtype=torch.int16, device=device)
    else:
        bufs["p"] = torch.empty(total, dtype=tdt[p_kind.split("_")[0]], device=device)
    mv = bufs["p"].dtype if scaled or p_kind in ("bf16", "f16") else torch.float32
    bufs["m"] = torch.zeros(total, dtype=mv, device=device)
    bufs["v"] = torch.zeros(total, dtype=mv, device=device)
    bufs["g"] = torch.empty(total, dtype=tdt[g_dtype], device=device)
    out_type = _out_type(p_out)
    if out_type is not None:
        bufs["p_out"] = torch.zeros(total, dtype=tdt[out_type], device=device)
    scale = float(g_std * g_multiplier)
    p_mul = 1.0 / scaled_p_scale(p_kind) if scaled else 1.0
    for lo in range(0, total, chunk):
        hi = min(total, lo + chunk)
        n = hi - lo
        tmp = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if p_mul != 1.0:
            tmp.mul_(p_mul)
        bufs["p"][lo:hi].copy_(tmp)
        tmp = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        tmp.mul_(scale)
        bufs["g"][lo:hi].copy_(tmp)
        if "rem" in bufs:
            r = torch.randint(-32768, 32768, (n,), generator=gen, device=device,
                              dtype=torch.int32)
            bufs["rem"][lo:hi].copy_(r)
        del tmp
    return bufs


def scaled_p_scale(p_kind: str) -> float:
    """The param scale of ``device_flat``'s scaled-state p (a power of two)."""
    return 2.0 ** -_F16_SHIFT["p"] if p_kind == "f16_scaled" else 1.0


def split_views(buf, sizes: Sequence[int]):
    """Contiguous views of a flat buffer, one per tensor size."""
    views = []
    off = 0
    for n in sizes:
        views.append(buf[off:off + n])
        off += n
    return views
