"""Helpers for the GPU parity tests: seeded host inputs -> device buffers
(optionally at odd element offsets), read-back, and comparison with the
oracle.  Only marshalling; no update arithmetic."""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

import adamw_optimizer_step_tensor_amd as A
from oracle import HParams, OracleTensor
from workloads import HostTensor

ROLES = ("p", "rem", "m", "v", "g", "p_out", "scales")


def torch_mod():
    import torch

    return torch


def np_to_dev(a: np.ndarray, role: str, offset: int = 0, pad: int = 8):
    """Device copy of a host array placed ``offset`` elements into a fresh
    allocation (to test unaligned bases)."""
    torch = torch_mod()
    if a.dtype in (np.float32, np.float16, np.int16):
        t = torch.from_numpy(a)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        raise TypeError(a.dtype)
    buf = torch.zeros(a.size + offset + pad, dtype=t.dtype, device="cuda")
    view = buf[offset:offset + a.size]
    view.copy_(t)
    return view


def dev_to_np(t) -> np.ndarray:
    torch = torch_mod()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


class DeviceSet:
    """Device buffers mirroring a list of HostTensor."""

    def __init__(self, host: Sequence[HostTensor], offsets: Optional[List[Dict[str, int]]] = None):
        self.tensors = []
        for i, h in enumerate(host):
            off = offsets[i] if offsets else {}
            d = {}
            for role in ROLES:
                a = getattr(h, role)
                if a is not None:
                    d[role] = np_to_dev(a, role, off.get(role, 0))
            self.tensors.append(d)

    def readback(self) -> List[HostTensor]:
        out = []
        for d in self.tensors:
            vals = {r: (dev_to_np(d[r]) if r in d else None) for r in ROLES}
            out.append(HostTensor(vals["p"], vals["m"], vals["v"], vals["g"], vals["p_out"],
                                  vals["rem"], vals["scales"]))
        return out

    def set_grad(self, i: int, idx: int, value: float):
        g = self.tensors[i]["g"]
        g[idx] = value


def oracle_tensors(host: Sequence[HostTensor]) -> List[OracleTensor]:
    return [OracleTensor(h.p, h.m, h.v, h.g, h.p_out, h.rem, h.scales) for h in host]


def copies(host: Sequence[HostTensor]) -> List[HostTensor]:
    return [h.copy() for h in host]


def assert_bitwise(got: Sequence[HostTensor], want: Sequence[HostTensor],
                   roles=("p", "rem", "m", "v", "p_out", "scales"),
                   ctx=""):
    """Bit-for-bit equality; NaNs compare as NaN regardless of payload (the
    CPU and the GPU make different default NaN bits)."""
    for k, (g, w) in enumerate(zip(got, want)):
        for r in roles:
            a, b = getattr(g, r), getattr(w, r)
            if a is None and b is None:
                continue
            assert a is not None and b is not None, (ctx, k, r)
            if a.dtype == np.float32:
                nan = np.isnan(a) & np.isnan(b)
                bad = (a.view(np.uint32) != b.view(np.uint32)) & ~nan
            elif a.dtype == np.float16:
                nan = np.isnan(a) & np.isnan(b)
                bad = (a.view(np.uint16) != b.view(np.uint16)) & ~nan
            elif a.dtype == np.uint16:  # bf16 bits
                fa = (a.astype(np.uint32) << 16).view(np.float32)
                fb = (b.astype(np.uint32) << 16).view(np.float32)
                nan = np.isnan(fa) & np.isnan(fb)
                bad = (a != b) & ~nan
            else:
                bad = a != b
            if bad.any():
                i = int(np.nonzero(bad)[0][0])
                raise AssertionError(f"{ctx} tensor {k} {r}: {int(bad.sum())} of {a.size} differ; "
                                     f"first at {i}: got {a[i]!r} want {b[i]!r}")


def assert_within_tolerance(got, want, roles=("p", "m", "v")):
    """The contract's floating-point bar: max |d| <= 1e-6 * max(1, |x|)."""
    for g, w in zip(got, want):
        for r in roles:
            a, b = getattr(g, r), getattr(w, r)
            if a is None or a.dtype != np.float32:
                continue
            fin = np.isfinite(b)
            d = np.abs(a[fin].astype(np.float64) - b[fin])
            assert np.all(d <= 1e-6 * np.maximum(1.0, np.abs(b[fin]))), r


def hp_pair(beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, mode=1, bc=1):
    """The same hyperparameters for the library and for the oracle."""
    return A.AdamHParams(beta1, beta2, eps, wd, mode, bc), HParams(beta1, beta2, eps, wd, mode, bc)


def _short(a: Optional[np.ndarray]) -> Optional[str]:
    if a is None:
        return None
    return {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16",
            np.dtype(np.float16): "f16"}[a.dtype]


def desc_for(host: Sequence[HostTensor], **kw):
    h = host[0]
    if h.rem is not None:
        p = "bf16_rem"
    elif h.scales is not None:
        p = _short(h.p) + "_scaled"
    else:
        p = _short(h.p)  # "f32", or 16-bit state "bf16" / "f16"
    return A.make_desc(g=_short(h.g), p=p, p_out=_short(h.p_out), **kw)
