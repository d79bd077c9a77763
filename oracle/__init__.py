"""Oracle for the fused multi-tensor Adam / AdamW step (CPU, fp32, scalar).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and never imports it.

The element arithmetic lives in ``adam_oracle.c`` (plain C, one IEEE binary32
operation per printed operation, no fused multiply-add).  This module loads
it with ctypes and adds the step-level rules around one call:

* the capturable call returns at once when the noop flag is 1, and then the
  step counter does not move either (apex patch "Enhance Distributed Fused
  Adam (#1794)": DistAdamCapturableFunctor::operator() returns on noop == 1,
  and DistributedFusedAdam.step() adds ``noop != 1`` to the counter);
* otherwise the counter is incremented before the update, so the first
  update uses t = 1 (apex distributed_fused_adam.py, step());
* a group with no elements still advances its counter (TransformerEngine PR
  "Advance FusedAdam step counter for empty param groups", section "Fix").

Arrays are numpy: fp32 as ``float32``, fp16 as ``float16``, bf16 as raw
``uint16`` bits, the remainders as ``int16``.  Scaled optimizer state (apex
distributed_fused_adam.py, ``_local_step_with_scaled_states``) keeps p, m and
v as bf16 bits or fp16 with three float32 scales per tensor.

Every function is pinned by ``tests/test_oracle_pins.py`` to values fixed by
the pages or by mathematics (closed forms, exact rational arithmetic,
exhaustive encodings, a float64 library optimizer, a float64 shadow with a
forward error bound); ``tests/test_oracle_mutants.py`` plants plausible
mistakes in copies of the C source and checks that the pins catch each one.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "liboracle.so")


@dataclass
class HParams:
    """Per-group hyperparameters; defaults are apex's constructor defaults
    (apex distributed_fused_adam.py, DistributedFusedAdam.__init__)."""

    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    mode: int = 1  # 0 = L2, 1 = AdamW
    bias_correction: int = 1


@dataclass
class OracleTensor:
    """One tensor of a group.  For fp32 params ``p``, ``m``, ``v`` are float32
    and ``rem`` and ``scales`` are None; for 16-bit state ``p``, ``m``, ``v``
    are all bf16 bits (uint16) or all float16, without ``rem`` or
    ``scales``; for remainder params ``p`` is bf16 bits (uint16), ``rem``
    int16 and ``m``, ``v`` float32; for scaled state ``p``, ``m``, ``v`` are
    bf16 bits (uint16) or float16 and ``scales`` is float32[3] (param,
    exp_avg, exp_avg_sq).  ``g`` is float32, bf16 bits (uint16) or float16.
    ``p_out`` is float32 (fp32 or 16-bit state only), bf16 bits (uint16),
    float16 or None."""

    p: np.ndarray
    m: np.ndarray
    v: np.ndarray
    g: np.ndarray
    p_out: Optional[np.ndarray] = None
    rem: Optional[np.ndarray] = None
    scales: Optional[np.ndarray] = None

    @property
    def numel(self) -> int:
        return int(self.p.size)


# element type codes of adam_oracle.c
F32, BF16, F16 = 0, 1, 2


def type_code(a: np.ndarray) -> int:
    """float32 -> F32, uint16 (bf16 bits) -> BF16, float16 -> F16."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"unsupported element type {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


class Oracle:
    """The oracle loaded from one compiled copy of ``adam_oracle.c``."""

    def __init__(self, path: str = LIBRARY_PATH):
        lib = ctypes.CDLL(path)
        f32, i32, i64, vp = ctypes.c_float, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_pow_int.argtypes = [ctypes.c_double, i32]
        lib.oracle_pow_int.restype = ctypes.c_double
        lib.oracle_bias_corrections.argtypes = [f32, f32, i32, i32, f32p, f32p]
        lib.oracle_bias_corrections.restype = None
        lib.oracle_bf16_rne_array.argtypes = [vp, vp, i64]
        lib.oracle_bf16_rne_array.restype = None
        lib.oracle_rem_encode_array.argtypes = [vp, vp, vp, i64]
        lib.oracle_rem_encode_array.restype = None
        lib.oracle_rem_decode_array.argtypes = [vp, vp, vp, i64]
        lib.oracle_rem_decode_array.restype = None
        lib.oracle_f16_rne_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_rne_array.restype = None
        lib.oracle_f16_to_f32_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_to_f32_array.restype = None
        common = [f32, f32, f32, f32, f32, i32, f32, f32, f32]
        lib.oracle_adam_f32.argtypes = [vp, vp, vp, vp, i32, vp, i32, i64, *common]
        lib.oracle_adam_f32.restype = None
        lib.oracle_adam_state16.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i64, *common]
        lib.oracle_adam_state16.restype = None
        lib.oracle_adam_remainder.argtypes = [vp, vp, vp, vp, vp, i32, vp, i64, *common]
        lib.oracle_adam_remainder.restype = None
        lib.oracle_adam_scaled.argtypes = [vp, vp, vp, i32, vp, vp, i32, vp, i32, i64, *common]
        lib.oracle_adam_scaled.restype = ctypes.c_int
        lib.oracle_scaled_state_limit.argtypes = [i32]
        lib.oracle_scaled_state_limit.restype = f32
        lib.oracle_rescale_store.argtypes = [vp, vp, i64, i32]
        lib.oracle_rescale_store.restype = f32
        lib.oracle_acc_size.argtypes = []
        lib.oracle_acc_size.restype = ctypes.c_size_t
        lib.oracle_acc_clear.argtypes = [vp]
        lib.oracle_acc_clear.restype = None
        lib.oracle_acc_add_squares.argtypes = [vp, vp, i32, i64]
        lib.oracle_acc_add_squares.restype = None
        lib.oracle_acc_merge.argtypes = [vp, vp]
        lib.oracle_acc_merge.restype = None
        lib.oracle_acc_value.argtypes = [vp]
        lib.oracle_acc_value.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    # -- scalar pieces ------------------------------------------------------

    def pow_int(self, beta: float, t: int) -> float:
        """beta**t in double by binary exponentiation (1 for t <= 0)."""
        return self.lib.oracle_pow_int(float(beta), int(t))

    def bias_corrections(self, beta1: float, beta2: float, t: int,
                         bias_correction: int):
        """(bc1, bc2) as float32: 1 - beta^t rounded once to float, or 1 when
        bias correction is off."""
        b1, b2 = ctypes.c_float(), ctypes.c_float()
        self.lib.oracle_bias_corrections(beta1, beta2, int(t), int(bias_correction),
                                         ctypes.byref(b1), ctypes.byref(b2))
        return np.float32(b1.value), np.float32(b2.value)

    def bf16_rne(self, x: np.ndarray) -> np.ndarray:
        """float32 array -> bf16 bits (uint16), round to nearest even."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_bf16_rne_array(_ptr(x), _ptr(out), x.size)
        return out

    def f16_rne(self, x: np.ndarray) -> np.ndarray:
        """float32 array -> float16 (round to nearest even, IEEE overflow and
        subnormals)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f16_rne_array(_ptr(x), _ptr(out), x.size)
        return out.view(np.float16)

    def f16_to_f32(self, h: np.ndarray) -> np.ndarray:
        """float16 array -> float32 (exact)."""
        h = np.ascontiguousarray(h, dtype=np.float16)
        out = np.empty(h.shape, dtype=np.float32)
        self.lib.oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
        return out

    def scaled_state_limit(self, state_dtype) -> np.float32:
        """Half the largest finite value of the state type (bf16 bits as
        uint16, or float16), as float32."""
        code = type_code(np.empty(0, dtype=state_dtype))
        return np.float32(self.lib.oracle_scaled_state_limit(code))

    def scale_state(self, x: np.ndarray, state_dtype):
        """float32 values -> (scaled 16-bit values, float32 scale), as apex's
        _apply_state_scale followed by the copy into the state type."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        assert x.size > 0
        out = np.empty(x.shape, dtype=np.uint16)
        code = type_code(np.empty(0, dtype=state_dtype))
        scale = self.lib.oracle_rescale_store(_ptr(x), _ptr(out), x.size, code)
        return out.view(state_dtype), np.float32(scale)

    def unscale_state(self, x: np.ndarray, scale) -> np.ndarray:
        """Scaled 16-bit values -> float32: the copy to float, times the
        scale (one float multiplication)."""
        wide = self.f16_to_f32(x) if x.dtype == np.float16 else \
            (x.astype(np.uint32) << 16).view(np.float32)
        return (wide * np.float32(scale)).astype(np.float32)

    def rem_encode(self, x: np.ndarray):
        """float32 array -> (bf16 bits uint16, remainder int16)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        hi = np.empty(x.shape, dtype=np.uint16)
        lo = np.empty(x.shape, dtype=np.int16)
        self.lib.oracle_rem_encode_array(_ptr(x), _ptr(hi), _ptr(lo), x.size)
        return hi, lo

    def rem_decode(self, bf16: np.ndarray, rem: np.ndarray) -> np.ndarray:
        """(bf16 bits, int16 remainder) -> float32 master value."""
        bf16 = np.ascontiguousarray(bf16, dtype=np.uint16)
        rem = np.ascontiguousarray(rem, dtype=np.int16)
        out = np.empty(bf16.shape, dtype=np.float32)
        self.lib.oracle_rem_decode_array(_ptr(bf16), _ptr(rem), _ptr(out), bf16.size)
        return out

    # -- one tensor, one call ------------------------------------------------

    def update_tensor(self, t: OracleTensor, hp: HParams, lr: float, bc1, bc2,
                      grad_scale: float, lo: int = 0, hi: Optional[int] = None) -> None:
        """Applies the element update to elements [lo, hi) of one tensor."""
        n = t.numel if hi is None else hi
        count = n - lo
        if count <= 0:
            return
        g_type = type_code(t.g)
        out_type = F32 if t.p_out is None else type_code(t.p_out)
        scal = (float(lr), float(hp.beta1), float(hp.beta2), float(hp.eps),
                float(hp.weight_decay), int(hp.mode), float(bc1), float(bc2),
                float(grad_scale))
        g_ptr = _ptr(t.g) + t.g.dtype.itemsize * lo
        out_ptr = None if t.p_out is None else _ptr(t.p_out) + t.p_out.dtype.itemsize * lo
        if t.scales is not None:
            # the new scales depend on the whole tensor: no partial ranges
            assert lo == 0 and n == t.numel, "scaled state is updated whole"
            st = type_code(t.p)
            assert st in (BF16, F16) and t.m.dtype == t.p.dtype and t.v.dtype == t.p.dtype
            assert t.scales.dtype == np.float32 and t.scales.size == 3
            assert t.p_out is None or type_code(t.p_out) in (BF16, F16)
            rc = self.lib.oracle_adam_scaled(_ptr(t.p), _ptr(t.m), _ptr(t.v), st, _ptr(t.scales),
                                             g_ptr, g_type, out_ptr, out_type, count, *scal)
            if rc != 0:
                raise MemoryError("oracle_adam_scaled could not allocate its work buffers")
            return
        if t.rem is None and t.p.dtype != np.float32:
            # 16-bit state: p, m and v of one 16-bit type
            st = type_code(t.p)
            assert st in (BF16, F16) and t.m.dtype == t.p.dtype and t.v.dtype == t.p.dtype
            self.lib.oracle_adam_state16(_ptr(t.p) + 2 * lo, _ptr(t.m) + 2 * lo, _ptr(t.v) + 2 * lo, st,
                                         g_ptr, g_type, out_ptr, out_type, count, *scal)
            return
        m_ptr = _ptr(t.m) + 4 * lo
        v_ptr = _ptr(t.v) + 4 * lo
        if t.rem is None:
            assert t.p.dtype == np.float32 and t.m.dtype == np.float32 and t.v.dtype == np.float32
            self.lib.oracle_adam_f32(_ptr(t.p) + 4 * lo, m_ptr, v_ptr, g_ptr,
                                     g_type, out_ptr, out_type, count, *scal)
        else:
            assert t.p.dtype == np.uint16 and t.rem.dtype == np.int16
            assert t.p_out is None or out_type == BF16, "remainder param-out is the new bf16 param"
            self.lib.oracle_adam_remainder(_ptr(t.p) + 2 * lo, _ptr(t.rem) + 2 * lo,
                                           m_ptr, v_ptr, g_ptr, g_type, out_ptr,
                                           count, *scal)

    # -- gradient norm and clipping -------------------------------------------

    def new_accumulator(self):
        """An exact sum-of-squares accumulator, cleared."""
        acc = ctypes.create_string_buffer(self.lib.oracle_acc_size())
        self.lib.oracle_acc_clear(acc)
        return acc

    def accumulate_squares(self, total, grads: Sequence[np.ndarray], threads: int = 1) -> None:
        """Adds the squares of every element of the gradient arrays (float32,
        bf16 bits as uint16, or float16) to the accumulator ``total``, exactly.
        ``threads`` > 1 splits the work; the result does not depend on it."""
        jobs = []  # (array, lo, hi)
        for g in grads:
            g = np.ascontiguousarray(g)
            type_code(g)
            n = g.size
            per = max(1, -(-n // max(1, threads)))
            for lo in range(0, n, per):
                jobs.append((g, lo, min(n, lo + per)))
        accs = [self.new_accumulator() for _ in jobs]

        def run(k):
            g, lo, hi = jobs[k]
            self.lib.oracle_acc_add_squares(accs[k], _ptr(g) + g.dtype.itemsize * lo,
                                            type_code(g), hi - lo)

        if threads > 1 and len(jobs) > 1:
            from concurrent.futures import ThreadPoolExecutor

            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, range(len(jobs))))
        else:
            for k in range(len(jobs)):
                run(k)
        for a in accs:
            self.lib.oracle_acc_merge(total, a)

    def accumulator_value(self, total) -> float:
        """The accumulated sum rounded once to the nearest double."""
        return self.lib.oracle_acc_value(total)

    def grad_sumsq(self, grads: Sequence[np.ndarray], threads: int = 1) -> float:
        """Sum of the squares of every element of the gradient arrays,
        computed exactly and rounded once to double."""
        total = self.new_accumulator()
        self.accumulate_squares(total, grads, threads)
        return self.accumulator_value(total)

    @staticmethod
    def clip_grad_scale(sumsq: float, grad_scale: Optional[float], max_norm: float):
        """The clip / found-inf step in float32 (apex distributed_fused_adam.py:
        grad_norm multiplies the raw norm by the grad scale, clip_grad_norm
        scales the grad scale by min(1, max_norm / (norm + 1e-6)), step() sets
        found_inf when the norm is not finite).  Returns (norm, new grad
        scale, found_inf as 0/1); the grad scale is left as it is when
        found_inf or max_norm <= 0."""
        f32 = np.float32
        raw = f32(math.sqrt(sumsq)) if sumsq == sumsq else f32(np.nan)
        scale = f32(1.0) if grad_scale is None else f32(grad_scale)
        with np.errstate(over="ignore", invalid="ignore"):
            norm = f32(raw * scale)
        found_inf = not np.isfinite(norm)
        new_scale = scale
        if not found_inf and max_norm > 0:
            coef = f32(f32(max_norm) / f32(norm + f32(1e-6)))
            if coef > f32(1.0):
                coef = f32(1.0)
            new_scale = f32(scale * coef)
        return norm, new_scale, 1 if found_inf else 0

    # -- one group, one step: the counter and noop rules --------------------

    def group_step(self, tensors: Sequence[OracleTensor], hp: HParams, lr: float,
                   step: List[int], grad_scale: float = 1.0,
                   noop: Optional[int] = None) -> bool:
        """One optimizer step of one group.

        ``step`` is a one-element list holding the group's int32 counter,
        updated in place.  ``noop`` is None for the non-capturable call, else
        the device flag's value for the capturable call.  Returns True when
        the element update ran.
        """
        if hp.mode not in (0, 1):
            raise ValueError("mode must be 0 (L2) or 1 (AdamW)")
        if hp.bias_correction not in (0, 1):
            raise ValueError("bias_correction must be 0 or 1")
        if noop is not None and int(noop) == 1:
            return False
        step[0] = ((int(step[0]) + 1 + 2**31) % 2**32) - 2**31  # int32 wrap
        if sum(t.numel for t in tensors) == 0:
            return False
        bc1, bc2 = self.bias_corrections(hp.beta1, hp.beta2, step[0], hp.bias_correction)
        for t in tensors:
            self.update_tensor(t, hp, lr, bc1, bc2, grad_scale)
        return True


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from this directory's ``adam_oracle.c``."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY_PATH):
            from . import build as _build

            _build.build()
        _default = Oracle(LIBRARY_PATH)
    return _default
