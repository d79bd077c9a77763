"""Python binding of libadamw_mi355x.so: the fused multi-tensor Adam / AdamW
step on MI355X (gfx950).

Argument marshalling only.  Every step of the update runs in the HIP library
(``csrc/adam.hip``) behind the C ABI of ``include/adam.h``; the functions here
carry the same names and turn torch tensors (or raw device addresses) into
the C structs.  PyTorch provides device memory and streams, nothing else.
There is no fallback: if the library is missing, importing the binding's
functions raises.

Typical use (one handle per parameter group, built once; buffers must stay
allocated and in place)::

    import torch
    import adamw_optimizer_step_tensor_amd as A

    tensors = [dict(p=p, m=m, v=v, g=g) for p, m, v, g in group]     # fp32 p/m/v, bf16 g
    tl = A.adam_tl_build(tensors, A.make_desc(g="bf16"))
    hp = A.AdamHParams(beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, mode=1)
    step = A.HostStep(0)
    A.adam_step(tl, hp, 1.6e-3, step)                                  # host lr and counter

    # capturable: every scalar on the device, recordable into a HIP graph
    d_lr = torch.tensor([1.6e-3], device="cuda")
    d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_noop = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    d_scale = torch.ones(1, device="cuda")
    A.adam_grad_sumsq(tl, d_sumsq)                                     # local grad-norm^2
    A.adam_clip_grad_scale(d_sumsq, d_scale, max_norm=1.0, d_noop=d_noop)
    A.adam_step_capturable(tl, hp, d_lr, d_step, d_scale, d_noop)

16-bit state (p, m, v all bf16 or all fp16) uses ``make_desc(p="bf16")`` (or
``"f16"``) with the same ``adam_step`` / ``adam_step_capturable``; any
param-out type, fp32 included, goes with fp32 or 16-bit state.  Remainder
storage uses ``make_desc(p="bf16_rem")`` with an int16 ``rem`` per
tensor and ``adam_step_remainders`` (or ``..._capturable``); scaled 16-bit
state uses ``make_desc(p="f16_scaled")`` (or ``"bf16_scaled"``) with a
float32[3] ``scales`` per tensor and ``adam_step_scaled`` (or ``..._capturable``).

Two-buffer state (fp32, 16-bit or remainder storage): pass a second set of
p, m, v (and rem) per tensor as ``alternates``; each step reads one set and
writes the other, and the state lives in set ``step & 1``::

    alts = [dict(p=p2, m=m2, v=v2) for p2, m2, v2 in second_set]
    tl = A.adam_tl_build(tensors, A.make_desc(g="bf16"), alternates=alts)
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libadamw_mi355x.so")

ADAM_OK, ADAM_EINVAL, ADAM_EDTYPE, ADAM_ENOMEM, ADAM_EHIP, ADAM_ETOOBIG = 0, -1, -2, -3, -4, -5
DT_NONE, DT_F32, DT_BF16, DT_F16 = 0, 1, 2, 3

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class AdamTensor(ctypes.Structure):
    """adam_tensor"""
    _fields_ = [("p", c_vp), ("rem", c_vp), ("m", c_vp), ("v", c_vp), ("g", c_vp),
                ("p_out", c_vp), ("scales", c_vp), ("numel", c_i64)]


class AdamTlDesc(ctypes.Structure):
    """adam_tl_desc"""
    _fields_ = [("p", c_i32), ("g", c_i32), ("p_out", c_i32), ("with_remainders", c_i32),
                ("chunk_elems", c_i64), ("scaled_state", c_i32), ("dispatch_tiles", c_i32),
                ("scaled_passes", c_i32), ("scaled_wait_us", c_i32)]


class AdamHParams(ctypes.Structure):
    """adam_hparams (defaults: apex's constructor defaults)."""
    _fields_ = [("beta1", c_f32), ("beta2", c_f32), ("eps", c_f32), ("weight_decay", c_f32),
                ("mode", c_i32), ("bias_correction", c_i32)]

    def __init__(self, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, mode=1,
                 bias_correction=1):
        super().__init__(beta1, beta2, eps, weight_decay, mode, bias_correction)


class AdamTlStats(ctypes.Structure):
    """adam_tl_stats"""
    _fields_ = [("tensors", c_i64), ("nonempty", c_i64), ("chunks", c_i64), ("elements", c_i64),
                ("chunk_elems", c_i64), ("vector_tensors", c_i64), ("grid_blocks", c_i64),
                ("tile_elems", c_i32), ("block_threads", c_i32), ("bytes_per_elem", c_i32),
                ("device", c_i32), ("two_buffer", c_i32), ("pieces", c_i32),
                ("dispatch_tiles", c_i32), ("dispatches", c_i32), ("scaled_passes", c_i32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class AdamError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().adam_status_string(status).decode()} ({status})")


_lib = None

EXPORTED = ("adam_abi_version", "adam_status_string", "adam_tl_plan", "adam_tl_build",
            "adam_tl_plan_two_buffer", "adam_tl_build_two_buffer", "adam_tl_destroy", "adam_tl_info", "adam_step", "adam_step_capturable",
            "adam_step_remainders", "adam_step_remainders_capturable", "adam_step_scaled",
            "adam_step_scaled_capturable", "adam_grad_sumsq", "adam_clip_grad_scale", "adam_step_noalloc")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            f"{LIBRARY_PATH} is missing: build it with "
            "`python -m adamw_optimizer_step_tensor_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIBRARY_PATH)
    L.adam_abi_version.argtypes = []
    L.adam_abi_version.restype = c_i32
    L.adam_status_string.argtypes = [c_i32]
    L.adam_status_string.restype = ctypes.c_char_p
    L.adam_tl_plan.argtypes = [ctypes.POINTER(AdamTensor), c_i64, ctypes.POINTER(AdamTlDesc),
                               ctypes.POINTER(AdamTlStats)]
    L.adam_tl_plan.restype = c_i32
    L.adam_tl_build.argtypes = [ctypes.POINTER(AdamTensor), c_i64, ctypes.POINTER(AdamTlDesc), c_vp,
                                ctypes.POINTER(c_vp)]
    L.adam_tl_build.restype = c_i32
    L.adam_tl_plan_two_buffer.argtypes = [ctypes.POINTER(AdamTensor), ctypes.POINTER(AdamTensor), c_i64,
                                          ctypes.POINTER(AdamTlDesc), ctypes.POINTER(AdamTlStats)]
    L.adam_tl_plan_two_buffer.restype = c_i32
    L.adam_tl_build_two_buffer.argtypes = [ctypes.POINTER(AdamTensor), ctypes.POINTER(AdamTensor), c_i64,
                                           ctypes.POINTER(AdamTlDesc), c_vp, ctypes.POINTER(c_vp)]
    L.adam_tl_build_two_buffer.restype = c_i32
    L.adam_tl_destroy.argtypes = [c_vp]
    L.adam_tl_destroy.restype = None
    L.adam_tl_info.argtypes = [c_vp, ctypes.POINTER(AdamTlStats)]
    L.adam_tl_info.restype = c_i32
    L.adam_step.argtypes = [c_vp, ctypes.POINTER(AdamHParams), c_f32, ctypes.POINTER(c_i32), c_f32,
                            c_vp, c_vp]
    L.adam_step.restype = c_i32
    L.adam_step_remainders.argtypes = L.adam_step.argtypes
    L.adam_step_remainders.restype = c_i32
    L.adam_step_scaled.argtypes = L.adam_step.argtypes
    L.adam_step_scaled.restype = c_i32
    L.adam_step_capturable.argtypes = [c_vp, ctypes.POINTER(AdamHParams), c_vp, c_vp, c_vp, c_vp, c_vp]
    L.adam_step_capturable.restype = c_i32
    L.adam_step_remainders_capturable.argtypes = L.adam_step_capturable.argtypes
    L.adam_step_remainders_capturable.restype = c_i32
    L.adam_step_scaled_capturable.argtypes = L.adam_step_capturable.argtypes
    L.adam_step_scaled_capturable.restype = c_i32
    L.adam_grad_sumsq.argtypes = [c_vp, c_vp, c_i32, c_vp]
    L.adam_grad_sumsq.restype = c_i32
    L.adam_clip_grad_scale.argtypes = [c_vp, c_vp, c_f32, c_vp, c_vp, c_vp]
    L.adam_clip_grad_scale.restype = c_i32
    L.adam_step_noalloc.argtypes = [ctypes.POINTER(AdamTensor), c_i64, ctypes.POINTER(AdamTlDesc),
                                    ctypes.POINTER(AdamHParams), c_f32, ctypes.POINTER(c_i32), c_f32, c_vp, c_vp]
    L.adam_step_noalloc.restype = c_i32
    if L.adam_abi_version() != 6:
        raise ImportError("libadamw_mi355x.so has an unexpected ABI version")
    _lib = L
    return L


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------

def _addr(x) -> Optional[int]:
    """Device address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _get(t, key):
    if isinstance(t, dict):
        return t.get(key)
    return getattr(t, key, None)


def _numel(t) -> int:
    n = _get(t, "numel")
    if n is not None and not callable(n):
        return int(n)
    p = _get(t, "p")
    return 0 if p is None else int(p.numel())


def _check_tensor(x, name, dtypes, device_type="cuda"):
    import torch

    if not isinstance(x, torch.Tensor):
        return
    if x.device.type != device_type:
        raise ValueError(f"{name} must be a {device_type} tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {x.dtype}, expected one of {dtypes}")


def _tensor_array(tensors: Sequence, desc: AdamTlDesc):
    arr = (AdamTensor * max(1, len(tensors)))()
    torch_dtypes = None
    try:
        import torch

        f32, bf16, f16, i16 = torch.float32, torch.bfloat16, torch.float16, torch.int16
        # 16-bit buffers may also be int16 views of the raw bits
        torch_dtypes = {DT_F32: (f32,), DT_BF16: (bf16, i16), DT_F16: (f16, i16)}
    except ImportError:  # raw addresses only
        pass
    mv = DT_F32 if desc.p == DT_F32 or desc.with_remainders == 1 else desc.p
    for i, t in enumerate(tensors):
        n = _numel(t)
        if torch_dtypes is not None:
            _check_tensor(_get(t, "p"), "p", torch_dtypes.get(desc.p, ()))
            _check_tensor(_get(t, "m"), "m", torch_dtypes[mv])
            _check_tensor(_get(t, "v"), "v", torch_dtypes[mv])
            _check_tensor(_get(t, "g"), "g", torch_dtypes.get(desc.g, ()))
            if _get(t, "p_out") is not None:
                _check_tensor(_get(t, "p_out"), "p_out", torch_dtypes.get(desc.p_out, ()))
            if _get(t, "rem") is not None:
                _check_tensor(_get(t, "rem"), "rem", (torch.int16,))
            if _get(t, "scales") is not None:
                _check_tensor(_get(t, "scales"), "scales", torch_dtypes[DT_F32])
        arr[i] = AdamTensor(_addr(_get(t, "p")), _addr(_get(t, "rem")), _addr(_get(t, "m")),
                            _addr(_get(t, "v")), _addr(_get(t, "g")), _addr(_get(t, "p_out")),
                            _addr(_get(t, "scales")), n)
    return arr


def make_desc(*, g="f32", p="f32", p_out=None, chunk_elems=0, dispatch_tiles=0, scaled_passes=0,
              scaled_wait_us=0) -> AdamTlDesc:
    """Descriptor from short names: g in {"f32", "bf16", "f16"}; p in {"f32",
    "bf16", "f16" (16-bit p, m, v), "bf16_rem" (bf16 + int16 remainders, fp32
    m, v), "bf16_scaled", "f16_scaled" (scaled 16-bit p, m, v)}; p_out in
    {None, "f32", "bf16", "f16"}; dispatch_tiles: tiles per kernel dispatch
    (0: the most one dispatch carries); scaled_passes (scaled state): 0
    automatic, 1 one pass, 2 two passes; scaled_wait_us: the one-pass wait
    (0: default, -1: none)."""
    gd = {"f32": DT_F32, "bf16": DT_BF16, "f16": DT_F16}[g]
    pd, rem, scaled = {"f32": (DT_F32, 0, 0), "bf16": (DT_BF16, 0, 0), "f16": (DT_F16, 0, 0),
                       "bf16_rem": (DT_BF16, 1, 0),
                       "bf16_scaled": (DT_BF16, 0, 1), "f16_scaled": (DT_F16, 0, 1)}[p]
    od = {None: DT_NONE, "f32": DT_F32, "bf16": DT_BF16, "f16": DT_F16}[p_out]
    return AdamTlDesc(pd, gd, od, rem, int(chunk_elems), scaled, int(dispatch_tiles), int(scaled_passes),
                      int(scaled_wait_us))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != ADAM_OK:
        raise AdamError(status, what)


# ---------------------------------------------------------------------------
# The C ABI, one function each
# ---------------------------------------------------------------------------

def _alternate_array(alternates: Sequence, tensors: Sequence, desc: AdamTlDesc):
    """The second buffer set of a two-buffer handle: p, m, v (and rem) per
    tensor, numel taken from the tensor it pairs with."""
    if len(alternates) != len(tensors):
        raise ValueError("alternates must pair one-to-one with tensors")
    pairs = []
    for a, t in zip(alternates, tensors):
        pairs.append({"p": _get(a, "p"), "m": _get(a, "m"), "v": _get(a, "v"), "rem": _get(a, "rem"),
                      "numel": _numel(t)})
    return _tensor_array(pairs, desc)


def adam_tl_plan(tensors: Sequence, desc: AdamTlDesc, alternates: Optional[Sequence] = None) -> dict:
    """Host-only validation and planning; returns the statistics dict.  With
    ``alternates``: a two-buffer handle's plan (adam_tl_plan_two_buffer)."""
    arr = _tensor_array(tensors, desc)
    st = AdamTlStats()
    if alternates is None:
        _check(lib().adam_tl_plan(arr, len(tensors), ctypes.byref(desc), ctypes.byref(st)),
               "adam_tl_plan")
    else:
        alt = _alternate_array(alternates, tensors, desc)
        _check(lib().adam_tl_plan_two_buffer(arr, alt, len(tensors), ctypes.byref(desc), ctypes.byref(st)),
               "adam_tl_plan_two_buffer")
    return st.as_dict()


class TensorList:
    """Owns an adam_tl handle (and keeps its tensors referenced)."""

    def __init__(self, handle: int, tensors: Sequence, desc: AdamTlDesc):
        self.handle = handle
        self._tensors = list(tensors)  # keep the buffers alive
        self.desc = desc

    def info(self) -> dict:
        st = AdamTlStats()
        _check(lib().adam_tl_info(self.handle, ctypes.byref(st)), "adam_tl_info")
        return st.as_dict()

    def destroy(self):
        if self.handle:
            lib().adam_tl_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def adam_tl_build(tensors: Sequence, desc: AdamTlDesc, stream=None,
                  alternates: Optional[Sequence] = None) -> TensorList:
    """Builds a handle for one group (see include/adam.h).  ``tensors`` holds
    dicts or objects with p, m, v, g and optional rem / p_out / scales (torch
    tensors or int device addresses plus ``numel``).  ``alternates`` (one per
    tensor: p, m, v and rem in remainder mode) makes a two-buffer handle
    (adam_tl_build_two_buffer): the state then lives in set ``step & 1``,
    set 0 being ``tensors``."""
    arr = _tensor_array(tensors, desc)
    out = c_vp()
    s = _stream(stream) if len(tensors) and any(_numel(t) for t in tensors) else (stream or 0)
    if alternates is None:
        _check(lib().adam_tl_build(arr, len(tensors), ctypes.byref(desc), s, ctypes.byref(out)),
               "adam_tl_build")
        return TensorList(out.value, tensors, desc)
    alt = _alternate_array(alternates, tensors, desc)
    _check(lib().adam_tl_build_two_buffer(arr, alt, len(tensors), ctypes.byref(desc), s, ctypes.byref(out)),
           "adam_tl_build_two_buffer")
    return TensorList(out.value, list(tensors) + list(alternates), desc)


class HostStep:
    """A host int32 step counter (the non-capturable counter)."""

    def __init__(self, value: int = 0):
        self._c = c_i32(value)

    @property
    def value(self) -> int:
        return self._c.value

    @value.setter
    def value(self, v: int):
        self._c.value = v


def _step_args(tl, hp, lr, step: HostStep, grad_scale, d_grad_scale, stream):
    s = _stream(stream) if tl.info()["chunks"] else (0 if stream is None else _stream(stream))
    return (tl.handle, ctypes.byref(hp), float(lr), ctypes.byref(step._c), float(grad_scale),
            _addr(d_grad_scale), s)


def adam_step(tl: TensorList, hp: AdamHParams, lr: float, step: HostStep,
              grad_scale: float = 1.0, d_grad_scale=None, stream=None) -> None:
    """Non-capturable step of an fp32-param handle."""
    _check(lib().adam_step(*_step_args(tl, hp, lr, step, grad_scale, d_grad_scale, stream)),
           "adam_step")


def adam_step_remainders(tl: TensorList, hp: AdamHParams, lr: float, step: HostStep,
                         grad_scale: float = 1.0, d_grad_scale=None, stream=None) -> None:
    """Non-capturable step of a bf16 + int16-remainder handle."""
    _check(lib().adam_step_remainders(*_step_args(tl, hp, lr, step, grad_scale, d_grad_scale,
                                                  stream)), "adam_step_remainders")


def adam_step_scaled(tl: TensorList, hp: AdamHParams, lr: float, step: HostStep,
                     grad_scale: float = 1.0, d_grad_scale=None, stream=None) -> None:
    """Non-capturable step of a scaled 16-bit-state handle (each tensor's
    ``scales`` are read and replaced)."""
    _check(lib().adam_step_scaled(*_step_args(tl, hp, lr, step, grad_scale, d_grad_scale, stream)),
           "adam_step_scaled")


def adam_step_capturable(tl: TensorList, hp: AdamHParams, d_lr, d_step, d_grad_scale=None,
                         d_noop=None, stream=None) -> None:
    """Capturable step: lr (float32), step (int32), grad scale (float32) and
    noop flag (int32) are device tensors (or addresses)."""
    _check(lib().adam_step_capturable(tl.handle, ctypes.byref(hp), _addr(d_lr), _addr(d_step),
                                      _addr(d_grad_scale), _addr(d_noop), _stream(stream)),
           "adam_step_capturable")


def adam_step_remainders_capturable(tl: TensorList, hp: AdamHParams, d_lr, d_step,
                                    d_grad_scale=None, d_noop=None, stream=None) -> None:
    """Capturable step of a bf16 + int16-remainder handle (device scalars as
    adam_step_capturable)."""
    _check(lib().adam_step_remainders_capturable(tl.handle, ctypes.byref(hp), _addr(d_lr),
                                                 _addr(d_step), _addr(d_grad_scale), _addr(d_noop),
                                                 _stream(stream)),
           "adam_step_remainders_capturable")


def adam_step_scaled_capturable(tl: TensorList, hp: AdamHParams, d_lr, d_step,
                                d_grad_scale=None, d_noop=None, stream=None) -> None:
    """Capturable step of a scaled-state handle (device scalars as
    adam_step_capturable; a noop step leaves values and scales)."""
    _check(lib().adam_step_scaled_capturable(tl.handle, ctypes.byref(hp), _addr(d_lr), _addr(d_step),
                                             _addr(d_grad_scale), _addr(d_noop), _stream(stream)),
           "adam_step_scaled_capturable")


def adam_grad_sumsq(tl: TensorList, d_sumsq, accumulate: bool = False, stream=None) -> None:
    """*d_sumsq (device float64) = (accumulate ? *d_sumsq : 0) + the sum of
    squares of the handle's gradients."""
    _check(lib().adam_grad_sumsq(tl.handle, _addr(d_sumsq), 1 if accumulate else 0, _stream(stream)),
           "adam_grad_sumsq")


def adam_clip_grad_scale(d_sumsq, d_grad_scale=None, max_norm: float = 0.0, d_norm=None,
                         d_noop=None, stream=None) -> None:
    """Norm, found-inf flag and clipped grad scale from a sum of squares
    (device scalars; see include/adam.h)."""
    _check(lib().adam_clip_grad_scale(_addr(d_sumsq), _addr(d_grad_scale), float(max_norm),
                                      _addr(d_norm), _addr(d_noop), _stream(stream)),
           "adam_clip_grad_scale")



def adam_step_noalloc(tensors: Sequence, desc: AdamTlDesc, hp: AdamHParams, lr: float, step: HostStep,
                      grad_scale: float = 1.0, d_grad_scale=None, stream=None) -> None:
    """adam_step without a handle, for callers that cannot allocate device
    memory: the work table goes to the library's static device array (see
    include/adam.h; calls on one device must not overlap)."""
    arr = _tensor_array(tensors, desc)
    s = _stream(stream) if any(_numel(t) for t in tensors) else (0 if stream is None else _stream(stream))
    _check(lib().adam_step_noalloc(arr, len(tensors), ctypes.byref(desc), ctypes.byref(hp), float(lr),
                                   ctypes.byref(step._c), float(grad_scale), _addr(d_grad_scale), s),
           "adam_step_noalloc")
