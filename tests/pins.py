"""Pins for the oracle: checks against values fixed by the pages or by
mathematics, never against the oracle's own formulas retyped.

Each ``check_*`` takes an :class:`oracle.Oracle` and raises AssertionError on
a mismatch.  ``tests/test_oracle_pins.py`` runs them (some exhaustively) on
the real oracle; ``tests/test_oracle_mutants.py`` runs the quick forms on
copies of the oracle with planted mistakes and requires each copy to fail at
least one.

What pins what:
* bias correction           - exact rational arithmetic (decimal, 100 digits)
                              rounded to the nearest float by hand;
* first step, AdamW / L2 /  - closed forms: with zero moments the bias-
  no bias correction          corrected moments are g' and g'^2, so the step
                              is lr*(sign(g')/(1+eps/|g'|) [+ wd*p]);
* constant gradient         - closed form of the AdamW recurrence;
* zero gradient             - the AdamW decay recurrence, bitwise in float32;
* random multi-step runs    - float64 shadow of the equations, within a
                              forward error bound, and float64
                              torch.optim.Adam / AdamW (a library optimizer);
* bf16 round-to-nearest-even - torch's CPU float32 -> bfloat16 cast;
* remainder encoding        - the little-endian layout the pages' loader uses
                              (remainder = int16 element 0 of the fp32 word),
                              exact round trip, and the nearest-value property
                              of the stored bf16 half;
* noop flag, empty group    - the pages' step rules and the printed output of
                              the empty-group reproduction (tests/golden);
* gradient sum of squares   - math.fsum (a correctly rounded sum) of the
                              squares, closed forms, non-finite inputs;
* clip / found-inf step     - float64 torch.nn.utils.clip_grad_norm_;
* fp16 casts                - numpy's float32 -> float16 cast (round to
                              nearest even, IEEE overflow, subnormals) and
                              its exact float16 -> float32 widening;
* fp16 gradients / p_out    - the fp32 update of the exactly widened
                              gradient, numpy's cast of the new param;
* fp32 param-out            - the new param itself;
* 16-bit state (T bf16/fp16) - the pinned fp32 update of the widened values,
                              rounded to T by torch's / numpy's casts; the
                              param-out the library cast of the new T value;
* scaled 16-bit state       - the pages' own torch op sequence for the
                              unscale / rescale steps (aminmax, maximum, div,
                              reciprocal, where, mul, dtype casts) around the
                              pinned fp32 update; closed forms (zero tensors,
                              power-of-two scales); the largest stored value
                              sits at half the type's maximum; NaN
                              propagation.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from typing import Iterable, Optional

import numpy as np

import oracle as oracle_pkg
from oracle import HParams, Oracle, OracleTensor

F32_EPS = 2.0 ** -24  # unit roundoff of binary32


def f32(x) -> float:
    """The float32 value of x, as a Python float."""
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# Bias correction
# ---------------------------------------------------------------------------

def nearest_f32(d: Decimal) -> np.float32:
    """The float32 nearest to the exact decimal ``d`` (ties to even)."""
    guess = np.float32(float(d))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess,
             np.nextafter(guess, np.float32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Decimal(float(c)) - d)
        key = (dist, int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def exact_bias_correction(beta: float, t: int) -> Decimal:
    getcontext().prec = 100
    return Decimal(1) - Decimal(float(np.float32(beta))) ** t


def check_bias_corrections(o: Oracle, betas: Iterable[float] = (0.9, 0.95, 0.999, 0.5, 0.99999),
                           steps: Iterable[int] = tuple(range(1, 301)) + (1000, 4096, 12345, 100000,
                                                                           1000000, 2**31 - 1)):
    """bc = 1 - beta^t rounded once to float32 from the exact value.  The
    oracle may differ only when the exact value lies within its documented
    double-precision error (about t * 2^-52 relative to beta^t) of a float32
    rounding boundary."""
    getcontext().prec = 100
    for beta in betas:
        for t in steps:
            exact = exact_bias_correction(beta, t)
            want = nearest_f32(exact)
            for got in o.bias_corrections(beta, beta, t, 1):
                if got != want:
                    # only allowed next to a rounding boundary
                    pw = Decimal(float(np.float32(beta))) ** t
                    slack = pw * Decimal(2.0 ** -52) * (2 * t.bit_length() + 2)
                    lo, hi = sorted([Decimal(float(got)), Decimal(float(want))])
                    mid = (lo + hi) / 2
                    assert abs(exact - mid) <= slack, (beta, t, got, want)
    # bias correction off: both are 1 whatever t
    for t in (1, 2, 77):
        assert o.bias_corrections(0.9, 0.999, t, 0) == (np.float32(1), np.float32(1))
    # the second beta feeds the second correction
    bc1, bc2 = o.bias_corrections(0.5, 0.75, 3, 1)
    assert bc1 == np.float32(1 - 0.125) and bc2 == np.float32(1 - 0.421875)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def _tensor(p, g, *, p_out=False):
    n = len(p)
    return OracleTensor(p=np.array(p, np.float32), m=np.zeros(n, np.float32),
                        v=np.zeros(n, np.float32), g=np.array(g, np.float32),
                        p_out=np.zeros(n, np.uint16) if p_out else None)


def _first_step_inputs(seed: int, n: int = 4096):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    # magnitudes around eps and far from it, both signs
    g[:8] = np.array([1e-8, -1e-8, 3e-9, -5e-7, 2.0, -7.5, 1e-12, -1e-12], np.float32)
    return p, g


def check_first_step_adamw(o: Oracle, seed: int = 11):
    """t = 1, m = v = 0, AdamW: p1 = p - lr*(sign(x)/(1+eps/|x|) + wd*p) with
    x = g*s (the moments' bias corrections cancel exactly in real numbers)."""
    p, g = _first_step_inputs(seed)
    for lr, wd, s, eps, b1, b2 in [(1e-3, 0.01, 1.0, 1e-8, 0.9, 0.999),
                                   (1.6e-3, 0.1, 0.5, 1e-8, 0.9, 0.95),
                                   (1e-2, 0.0, 3.0, 1e-6, 0.8, 0.99)]:
        t = _tensor(p, g)
        step = [0]
        o.group_step([t], HParams(b1, b2, eps, wd, 1, 1), lr, step, s)
        assert step == [1]
        x = g.astype(np.float64) * f32(s)
        want = p.astype(np.float64) - f32(lr) * (np.sign(x) / (1 + f32(eps) / np.abs(x))
                                                + f32(wd) * p.astype(np.float64))
        tol = F32_EPS * np.maximum(np.abs(want), 1e-30) + 8 * F32_EPS * f32(lr) * (1 + f32(wd) * np.abs(p))
        err = np.abs(t.p.astype(np.float64) - want)
        assert np.all(err <= tol), float(np.max(err / tol))
        # first moments: m = (1-b1) x, v = (1-b2) x^2, each within a few roundings
        xm = (1 - f32(b1)) * x
        xv = (1 - f32(b2)) * x * x
        assert np.all(np.abs(t.m - xm) <= 3 * F32_EPS * np.abs(xm) + 1e-45)
        assert np.all(np.abs(t.v - xv) <= 4 * F32_EPS * np.abs(xv) + 1e-45)


def check_first_step_l2(o: Oracle, seed: int = 12):
    """t = 1, m = v = 0, L2: x = g*s + wd*p and p1 = p - lr*sign(x)/(1+eps/|x|)."""
    p, g = _first_step_inputs(seed)
    g[8:16] = 0.0  # pure decay gradient
    for lr, wd, s in [(1e-3, 0.01, 1.0), (1.6e-3, 0.1, 0.25)]:
        t = _tensor(p, g)
        o.group_step([t], HParams(0.9, 0.999, 1e-8, wd, 0, 1), lr, [0], s)
        x = g.astype(np.float64) * f32(s) + f32(wd) * p.astype(np.float64)
        want = p.astype(np.float64) - f32(lr) * np.sign(x) / (1 + f32(1e-8) / np.abs(x))
        tol = F32_EPS * np.abs(want) + 16 * F32_EPS * f32(lr)
        assert np.all(np.abs(t.p - want) <= tol)


def check_first_step_no_bias_correction(o: Oracle, seed: int = 13):
    """bias_correction = 0, t = 1, m = v = 0:
    p1 = p - lr*((1-b1) x / (sqrt(1-b2)|x| + eps) [+ wd p])."""
    p, g = _first_step_inputs(seed)
    for mode in (0, 1):
        b1, b2, eps, wd, lr = 0.9, 0.999, 1e-8, 0.05, 1e-3
        t = _tensor(p, g)
        o.group_step([t], HParams(b1, b2, eps, wd, mode, 0), lr, [0], 1.0)
        p64 = p.astype(np.float64)
        x = g.astype(np.float64) + (f32(wd) * p64 if mode == 0 else 0.0)
        u = (1 - f32(b1)) * x / (math.sqrt(1 - f32(b2)) * np.abs(x) + f32(eps))
        if mode == 1:
            u = u + f32(wd) * p64
        want = p64 - f32(lr) * u
        tol = F32_EPS * np.abs(want) + 16 * F32_EPS * f32(lr) * (np.abs(u) + 1e-30)
        assert np.all(np.abs(t.p - want) <= tol)


def check_constant_gradient_closed_form(o: Oracle, steps: int = 10, seed: int = 14):
    """AdamW with the same gradient every step: the corrected moments stay g
    and g^2, so p_t = a^t p0 - c (1 - a^t)/wd with a = 1 - lr wd and
    c = g/(|g| + eps); for wd = 0, p_t = p0 - t lr c."""
    rng = np.random.default_rng(seed)
    p0 = rng.standard_normal(1000).astype(np.float32)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    for wd, b1, b2 in [(0.01, 0.9, 0.999), (0.1, 0.9, 0.95), (0.0, 0.8, 0.9)]:
        lr, eps = f32(1e-3), f32(1e-8)
        t = _tensor(p0, g)
        step = [0]
        for _ in range(steps):
            o.group_step([t], HParams(b1, b2, eps, wd, 1, 1), lr, step, 1.0)
        assert step == [steps]
        c = g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
        if wd:
            a = 1 - lr * f32(wd)
            want = a ** steps * p0 - c * (1 - a ** steps) / f32(wd)
        else:
            want = p0 - steps * lr * c
        tol = steps * (F32_EPS * np.abs(want) + 64 * F32_EPS * lr)
        assert np.all(np.abs(t.p - want) <= tol), float(np.max(np.abs(t.p - want) / tol))


def check_zero_gradient(o: Oracle, steps: int = 20, seed: int = 15):
    """AdamW with g = 0: m and v stay 0, the moment term of the update is
    +0/(0+eps) = +0, so p follows p <- p - lr*(+0 + wd*p) bitwise in float32
    (the +0 matters only for p = -0).  With wd = 0 nothing changes at all."""
    rng = np.random.default_rng(seed)
    p0 = rng.standard_normal(777).astype(np.float32)
    p0[:4] = np.array([0.0, -0.0, 1e-40, -3e38], np.float32)
    lr, wd = np.float32(1.6e-3), np.float32(0.1)
    t = _tensor(p0, np.zeros(777, np.float32))
    want = p0.copy()
    step = [0]
    for _ in range(steps):
        o.group_step([t], HParams(0.9, 0.95, 1e-8, float(wd), 1, 1), float(lr), step, 1.0)
        want = (want - lr * (np.float32(0.0) + wd * want)).astype(np.float32)
        assert np.array_equal(t.p.view(np.uint32), want.view(np.uint32))
        assert not np.any(t.m) and not np.any(t.v)
    t = _tensor(p0, np.zeros(777, np.float32))
    o.group_step([t], HParams(0.9, 0.95, 1e-8, 0.0, 1, 1), float(lr), [0], 1.0)
    assert np.array_equal(t.p.view(np.uint32), p0.view(np.uint32))


# ---------------------------------------------------------------------------
# Multi-step: float64 shadow with a forward error bound, and torch.optim
# ---------------------------------------------------------------------------

def _shadow_run(p0, grads, lr, b1, b2, eps, wd, mode, bias_correction, s):
    """The update equations in float64 with exact bias corrections, and a
    first-order bound on how far a float32 evaluation can drift from them:
    each rounding contributes at most u = 2^-24 of the magnitude it rounds,
    and errors already present propagate through the same equations."""
    E = F32_EPS
    p = p0.astype(np.float64).copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    err_p = np.zeros_like(p)
    err_m = np.zeros_like(p)
    err_v = np.zeros_like(p)
    for k, g in enumerate(grads, start=1):
        g = g.astype(np.float64)
        gs = g * s
        x = gs + (wd * p if mode == 0 else 0.0)
        mag_x = np.abs(gs) + (np.abs(wd * p) if mode == 0 else 0.0)
        err_x = 3 * E * mag_x + (wd * err_p if mode == 0 else 0.0)
        new_m = b1 * m + (1 - b1) * x
        new_v = b2 * v + (1 - b2) * x * x
        err_m = b1 * err_m + (1 - b1) * err_x + 3 * E * (b1 * np.abs(m) + (1 - b1) * mag_x)
        err_v = b2 * err_v + (1 - b2) * (2 * mag_x * err_x + err_x ** 2) \
            + 4 * E * (b2 * v + (1 - b2) * mag_x ** 2)
        m, v = new_m, new_v
        bc1 = 1 - b1 ** k if bias_correction else 1.0
        bc2 = 1 - b2 ** k if bias_correction else 1.0
        mh, vh = m / bc1, v / bc2
        err_mh = err_m / bc1 + 2 * E * np.abs(mh)
        err_vh = err_v / bc2 + 2 * E * vh
        root = np.sqrt(vh)
        with np.errstate(divide="ignore", invalid="ignore"):
            lin = np.where(root > 0, 0.5 * err_vh / root, np.inf)
        err_root = np.minimum(lin, np.sqrt(err_vh)) + E * root
        d = root + eps
        err_d = err_root + E * d
        u = mh / d
        err_u = err_mh / d + np.abs(mh) * err_d / (d * np.maximum(d - err_d, d / 2)) + 2 * E * np.abs(u)
        if mode == 1:
            err_u = err_u + wd * err_p + 3 * E * (np.abs(u) + np.abs(wd * p))
            u = u + wd * p
        p = p - lr * u
        err_p = err_p + lr * err_u + 3 * E * (np.abs(p) + lr * np.abs(u))
    return p, m, v, err_p, err_m, err_v


def check_random_runs_vs_shadow(o: Oracle, trials: int = 40, steps: int = 10, seed: int = 16):
    """Random hyperparameters (betas near 1 and not, eps from 1e-12 to 1e-2,
    grad_scale != 1, both modes, bias correction on and off), 8 elements,
    fresh gradients each step, against the float64 shadow within twice its
    first-order error bound."""
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        b1 = f32(rng.choice([0.9, 0.5, 0.99, 0.0, 0.95]))
        b2 = f32(rng.choice([0.999, 0.95, 0.9999, 0.5, 0.0]))
        eps = f32(10.0 ** rng.uniform(-12, -2))
        wd = f32(rng.choice([0.0, 0.01, 0.1, 0.5]))
        lr = f32(10.0 ** rng.uniform(-4, -1))
        s = f32(rng.choice([1.0, 0.5, 2.0 ** -16, 3.0, 1.7]))
        mode = int(trial % 2)
        bc = int(rng.random() < 0.8)
        p0 = rng.standard_normal(8).astype(np.float32)
        gscale = 1.0 / s if s < 1e-3 else 1.0
        grads = [(rng.standard_normal(8) * 10.0 ** rng.uniform(-5, 0) * gscale).astype(np.float32)
                 for _ in range(steps)]
        t = _tensor(p0, grads[0])
        step = [0]
        hp = HParams(b1, b2, eps, wd, mode, bc)
        for g in grads:
            t.g[:] = g
            o.group_step([t], hp, lr, step, s)
        p, m, v, err_p, err_m, err_v = _shadow_run(p0, grads, lr, b1, b2, eps, wd, mode, bc, s)
        ctx = dict(trial=trial, b1=b1, b2=b2, eps=eps, wd=wd, lr=lr, s=s, mode=mode, bc=bc)
        assert np.all(np.abs(t.m - m) <= 2 * err_m + 1e-44), ctx
        assert np.all(np.abs(t.v - v) <= 2 * err_v + 1e-44), ctx
        assert np.all(np.abs(t.p - p) <= 2 * err_p), ctx
        # the bound is tight enough to mean something: far below the update
        assert np.all(err_p < 1e-3 * lr * steps + 1e-5 * np.abs(p)), ctx


def check_against_torch_optim(o: Oracle, steps: int = 10, seed: int = 17):
    """float64 torch.optim.AdamW equals mode 1 and torch.optim.Adam with
    weight_decay (decay added to the gradient) equals mode 0, in real
    arithmetic; the oracle's float32 result must agree within the float32
    error of 10 steps (1e-6 relative to max(1, |p|))."""
    import torch

    rng = np.random.default_rng(seed)
    for mode in (0, 1):
        for lr, b1, b2, eps, wd, s in [(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0),
                                       (1.6e-3, 0.9, 0.95, 1e-8, 0.1, 0.5)]:
            lr, b1, b2, eps, wd, s = map(f32, (lr, b1, b2, eps, wd, s))
            n = 512
            p0 = rng.standard_normal(n).astype(np.float32)
            grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(steps)]
            tp = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
            cls = torch.optim.AdamW if mode == 1 else torch.optim.Adam
            opt = cls([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
            t = _tensor(p0, grads[0])
            step = [0]
            for g in grads:
                tp.grad = torch.from_numpy(g.astype(np.float64) * s)
                opt.step()
                t.g[:] = g
                o.group_step([t], HParams(b1, b2, eps, wd, mode, 1), lr, step, s)
            ref = tp.detach().numpy()
            assert np.all(np.abs(t.p - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref))), (mode, lr)
            st = opt.state[tp]
            m_ref = st["exp_avg"].numpy()
            v_ref = st["exp_avg_sq"].numpy()
            assert np.all(np.abs(t.m - m_ref) <= 1e-5 * np.max(np.abs(m_ref)))
            assert np.all(np.abs(t.v - v_ref) <= 1e-5 * np.max(np.abs(v_ref)))


# ---------------------------------------------------------------------------
# Param-out and remainder encodings
# ---------------------------------------------------------------------------

def torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def special_f32_patterns() -> np.ndarray:
    """Bit patterns at every rounding edge of the bf16 cast and the
    remainder split: ties with even/odd kept bits, one below/above a tie,
    carries into the exponent, max finite, inf, NaN, zeros, denormals."""
    hs = np.array([0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7F, 0x7F7E,
                   0x7F80, 0x7FC0, 0x8000, 0x8001, 0xBF80, 0xBF81, 0xFF7F, 0xFF80, 0xFFC0,
                   0x4049, 0xC049], np.uint32)
    ls = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    pats = (hs[:, None] << 16 | ls[None, :]).ravel()
    return pats.astype(np.uint32)


def check_bf16_rne(o: Oracle, patterns: np.ndarray):
    """Finite and infinite inputs: bitwise equal to torch's cast.  NaN: stays
    NaN with its sign."""
    x = patterns.astype(np.uint32).view(np.float32)
    got = o.bf16_rne(x)
    want = torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    if nan.any():
        gn = got[nan].astype(np.uint32)
        assert np.all((gn & 0x7F80) == 0x7F80) and np.all((gn & 0x007F) != 0)
        assert np.array_equal(gn >> 15, patterns[nan].astype(np.uint32) >> 31)


def check_remainder_codec(o: Oracle, patterns: np.ndarray):
    """For every float32 pattern x:
    * decode(encode(x)) is x, bit for bit;
    * the remainder is int16 element 0 of x's little-endian storage (the
      pages' state-dict loader splits the fp32 word that way);
    * the bf16 half is a nearest bf16 to x, with ties away from zero (the
      decoder's "minus one when the remainder is negative" forces this);
    * decoding any (bf16, remainder) pair and encoding again returns it."""
    pats = patterns.astype(np.uint32)
    x = pats.view(np.float32)
    hi, lo = o.rem_encode(x)
    back = o.rem_decode(hi, lo)
    assert np.array_equal(back.view(np.uint32), pats)
    assert np.array_equal(lo, pats.view(np.int16).reshape(-1, 2)[:, 0])
    # nearest-value property on finite x whose bf16 half is finite
    b = (hi.astype(np.uint32) << 16).view(np.float32)
    ok = np.isfinite(x) & np.isfinite(b)
    xs, bs, his = x[ok].astype(np.float64), b[ok].astype(np.float64), hi[ok].astype(np.uint32)
    up = (((his + 1) & 0xFFFF) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    dn = (((his - 1) & 0xFFFF) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    dist = np.abs(xs - bs)
    with np.errstate(invalid="ignore"):
        for nb in (up, dn):
            fin = np.isfinite(nb) & (np.sign(nb) == np.sign(bs))
            assert np.all(dist[fin] <= np.abs(xs[fin] - nb[fin]))
    tie = dist * 2 == np.abs(np.where(np.abs(up) > np.abs(bs), up, dn) - bs)
    tie &= dist > 0
    assert np.all(np.abs(bs[tie]) > np.abs(xs[tie]))  # ties go away from zero
    # every (bf16, remainder) pair round-trips
    rng = np.random.default_rng(0)
    hb = rng.integers(0, 65536, size=4096).astype(np.uint16)
    rm = rng.integers(-32768, 32768, size=4096).astype(np.int16)
    h2, r2 = o.rem_encode(o.rem_decode(hb, rm))
    assert np.array_equal(h2, hb) and np.array_equal(r2, rm)


def _layout_decode(bf16: np.ndarray, rem: np.ndarray) -> np.ndarray:
    """fp32 master from the storage layout: little-endian int16 pair
    (remainder, bf16 - [remainder < 0])."""
    pair = np.empty((bf16.size, 2), np.int16)
    pair[:, 0] = rem
    pair[:, 1] = (bf16.astype(np.int32) - (rem < 0)).astype(np.uint16).view(np.int16)
    return pair.reshape(-1).view(np.float32)


def check_param_out_and_remainder_update(o: Oracle, seed: int = 18):
    """p_out is torch's bf16 cast of the new fp32 param.  The remainder-mode
    update equals the fp32 update of the decoded master (layout decode), and
    stores the new master in the same layout; its p_out is the new bf16."""
    rng = np.random.default_rng(seed)
    n = 2053
    p0 = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g_bf16 = torch_bf16_bits(g)
    hp = HParams(0.9, 0.95, 1e-8, 0.1, 1, 1)
    # fp32 params with bf16 grads and bf16 p_out
    t = OracleTensor(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g_bf16.copy(),
                     np.zeros(n, np.uint16))
    step = [0]
    for _ in range(3):
        o.group_step([t], hp, 1.6e-3, step, 1.0)
        assert np.array_equal(t.p_out, torch_bf16_bits(t.p))
    # the bf16 grad is widened exactly: same result as the widened fp32 grad
    g_wide = (g_bf16.astype(np.uint32) << 16).view(np.float32)
    t32 = OracleTensor(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g_wide.copy())
    step = [0]
    for _ in range(3):
        o.group_step([t32], hp, 1.6e-3, step, 1.0)
    assert np.array_equal(t32.p.view(np.uint32), t.p.view(np.uint32))
    # remainder params
    hb = torch_bf16_bits(p0)
    rm = rng.integers(-32768, 32768, size=n).astype(np.int16)
    master = _layout_decode(hb, rm)
    tr = OracleTensor(hb.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g_bf16.copy(),
                      np.zeros(n, np.uint16), rm.copy())
    tf = OracleTensor(master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g_bf16.copy())
    sr, sf = [0], [0]
    for _ in range(4):
        o.group_step([tr], hp, 1.6e-3, sr, 1.0)
        o.group_step([tf], hp, 1.6e-3, sf, 1.0)
        assert np.array_equal(_layout_decode(tr.p, tr.rem).view(np.uint32), tf.p.view(np.uint32))
        assert np.array_equal(tr.m.view(np.uint32), tf.m.view(np.uint32))
        assert np.array_equal(tr.v.view(np.uint32), tf.v.view(np.uint32))
        assert np.array_equal(tr.p_out, tr.p)
        # stored bf16 is within half a bf16 ulp of the master
        b = (tr.p.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        half_ulp = np.abs(b) * 2.0 ** -8
        assert np.all(np.abs(tf.p - b) <= half_ulp)
    # lr = 0 leaves the master as it is; masters exactly halfway between two
    # bf16 values (low half 0x8000) with an even high half must keep the
    # stored (ties-away) bf16 in p_out, which differs from an RNE cast
    highs = np.array([0x3F80, 0x4000, 0xBF80, 0xC120], np.uint16)
    rem_tie = np.full(4, -32768, np.int16)  # low half 0x8000
    stored = (highs + 1).astype(np.uint16)  # decode subtracts one: master high = highs
    tq = OracleTensor(stored.copy(), np.zeros(4, np.float32), np.zeros(4, np.float32),
                      np.full(4, 1e-3, np.float32), np.zeros(4, np.uint16), rem_tie.copy())
    o.group_step([tq], HParams(0.9, 0.95, 1e-8, 0.0, 1, 1), 0.0, [0], 1.0)
    assert np.array_equal(tq.p, stored) and np.array_equal(tq.rem, rem_tie)
    assert np.array_equal(tq.p_out, stored)


# ---------------------------------------------------------------------------
# Step rules
# ---------------------------------------------------------------------------

def check_noop_and_counter(o: Oracle, seed: int = 19):
    """Capturable call with noop == 1: every buffer and the counter stay bit-
    identical.  Any other flag value runs the step and advances the counter
    (the pages skip on == 1 and advance on != 1)."""
    rng = np.random.default_rng(seed)
    p0 = rng.standard_normal(100).astype(np.float32)
    g = (rng.standard_normal(100) * 1e-3).astype(np.float32)
    g[5] = np.inf
    t = _tensor(p0, g, p_out=True)
    t.m[:] = 1e-4
    t.v[:] = 1e-8
    before = [a.copy() for a in (t.p, t.m, t.v, t.p_out)]
    step = [7]
    ran = o.group_step([t], HParams(), 1e-3, step, 1.0, noop=1)
    assert not ran and step == [7]
    for a, b in zip((t.p, t.m, t.v, t.p_out), before):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    t.g[5] = 0.0
    for flag, want in ((0, 8), (2, 9), (-1, 10)):
        assert o.group_step([t], HParams(), 1e-3, step, 1.0, noop=flag)
        assert step == [want]
    # an infinite gradient with noop == 0 propagates (no masking in the update)
    t.g[5] = np.inf
    o.group_step([t], HParams(), 1e-3, step, 1.0, noop=0)
    assert not np.isfinite(t.p[5]) and np.all(np.isfinite(np.delete(t.p, 5)))


def check_empty_group_counter(o: Oracle, golden_steps):
    """Three steps over one populated and one empty group leave both counters
    at the value the reproduction on the pages prints for the fixed loop, for
    the host counter and for the capturable (flag) path."""
    for noop in (None, 0):
        groups = [[_tensor(np.ones(4, np.float32), np.full(4, 1e-3, np.float32))], []]
        steps = [[0], [0]]
        for _ in range(3):
            for grp, st in zip(groups, steps):
                o.group_step(grp, HParams(), 1e-3, st, 1.0, noop=noop)
        assert [s[0] for s in steps] == list(golden_steps)


# ---------------------------------------------------------------------------
# Gradient sum of squares and the clip step
# ---------------------------------------------------------------------------

def _fsum_squares(values) -> float:
    return math.fsum(float(x) * float(x) for x in values)


def check_grad_sumsq(o: Oracle, n: int = 20001, seed: int = 40):
    """The oracle's sum of squares is the correctly rounded exact sum:
    equal to math.fsum of the (exact, double) squares, for values spread over
    the whole float range, split over arrays and threads, and for bf16."""
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-44, 37, n)).astype(np.float32)
    g[:6] = np.array([0.0, -0.0, 1e-45, 3.4e38, -1.0, 2.0 ** -149], np.float32)
    want = _fsum_squares(g)
    assert o.grad_sumsq([g]) == want
    assert o.grad_sumsq([g[:7], g[7:1000], g[1000:]], threads=3) == want
    gb = torch_bf16_bits(g[:5000])
    wide = (gb.astype(np.uint32) << 16).view(np.float32)
    assert o.grad_sumsq([gb]) == _fsum_squares(wide)
    # many equal values: a carry-heavy exact case with a closed form
    c = np.full(70000, 0.75, np.float32)
    assert o.grad_sumsq([c], threads=4) == 70000 * 0.5625
    ones = np.ones(1 << 20, np.float32)
    assert o.grad_sumsq([ones]) == float(1 << 20)
    # exact ties between two doubles round to the even one:
    # 2^52 + 2^52 + 1 = 2^53 + 1 -> 2^53;  2^53 + 3 -> 2^53 + 4
    big = np.float32(2.0 ** 26)
    assert o.grad_sumsq([np.array([big, big, 1.0], np.float32)]) == 2.0 ** 53
    assert o.grad_sumsq([np.array([big, big, 1.0, 1.0, 1.0], np.float32)]) == 2.0 ** 53 + 4
    assert _fsum_squares([big, big, 1.0, 1.0, 1.0]) == 2.0 ** 53 + 4
    # non-finite values, alone and after a threaded split
    assert o.grad_sumsq([]) == 0.0
    h = ones.copy()
    h[12345] = np.inf
    assert o.grad_sumsq([h], threads=4) == np.inf
    h[777] = np.nan
    assert np.isnan(o.grad_sumsq([h], threads=4))


def check_clip_grad_scale(o: Oracle, seed: int = 41):
    """Norm and clip factor agree with float64 torch.nn.utils.clip_grad_norm_
    on the scaled gradients; below the threshold the scale is untouched;
    a non-finite norm raises found_inf and leaves the scale; max_norm <= 0
    does not clip."""
    import torch

    rng = np.random.default_rng(seed)
    for trial in range(12):
        g = (rng.standard_normal(1000) * 10.0 ** rng.uniform(-4, 2)).astype(np.float32)
        s = f32(rng.choice([1.0, 0.5, 2.0 ** -16, 3.0]))
        max_norm = f32(10.0 ** rng.uniform(-3, 2))
        norm, new_s, found = o.clip_grad_scale(o.grad_sumsq([g]), s, max_norm)
        assert found == 0
        t = torch.nn.Parameter(torch.zeros(1000, dtype=torch.float64))
        t.grad = torch.from_numpy(g.astype(np.float64) * s)
        before = t.grad.clone()
        total = float(torch.nn.utils.clip_grad_norm_([t], float(max_norm)))
        factor = float((t.grad / before)[np.argmax(np.abs(g))])
        assert abs(float(norm) - total) <= 1e-6 * total, (trial, norm, total)
        assert abs(float(new_s) / float(s) - factor) <= 2e-6 * factor, (trial, new_s, s, factor)
        if total < float(max_norm) * (1 - 1e-5):
            assert new_s == np.float32(s)
    norm, new_s, found = o.clip_grad_scale(4.0, 1.0, 1.0)
    assert norm == np.float32(2.0) and new_s == np.float32(1.0) / np.float32(np.float32(2.0) + np.float32(1e-6))
    for bad in (np.inf, np.nan):
        norm, new_s, found = o.clip_grad_scale(bad, 0.5, 1.0)
        assert found == 1 and new_s == np.float32(0.5) and not np.isfinite(norm)
    norm, new_s, found = o.clip_grad_scale(1e6, 0.25, 0.0)
    assert found == 0 and new_s == np.float32(0.25) and norm == np.float32(1000.0 * 0.25)


# ---------------------------------------------------------------------------
# fp16 casts, fp16 gradients and param-out
# ---------------------------------------------------------------------------

def special_f16_edges() -> np.ndarray:
    """float32 bit patterns at the binary16 cast's edges: the overflow
    threshold 65520 and its neighbours, the largest finite 65504, the normal /
    subnormal boundary 2^-14, the smallest subnormal 2^-24 and the underflow
    tie 2^-25, ties with even and odd kept bits in both ranges, signed
    zeros, infinities, NaNs."""
    vals = [65504.0, 65519.996, 65520.0, 65520.004, 65535.0, 65536.0, 1e10,
            2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), 2.0 ** -24, 2.0 ** -25,
            2.0 ** -25 * (1 + 2.0 ** -20), 3 * 2.0 ** -25, 5 * 2.0 ** -25, 2.0 ** -26,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -20,
            2.0 ** -15 + 2.0 ** -25, 2.0 ** -15 + 3 * 2.0 ** -25, 0.1, 1.0 / 3.0, 1e-7]
    x = np.array(vals + [-v for v in vals], np.float32)
    extra = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000,
                      0xFFC00001, 0x7F800001, 0x00000001, 0x807FFFFF], np.uint32)
    pats = np.concatenate([x.view(np.uint32), extra])
    return np.concatenate([pats, pats + 1, pats - 1]).astype(np.uint32)


def check_f16_rne(o: Oracle, patterns: np.ndarray):
    """Finite and infinite inputs: bitwise equal to numpy's float32 ->
    float16 cast.  NaN: stays NaN with its sign."""
    x = patterns.astype(np.uint32).view(np.float32)
    got = o.f16_rne(x).view(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    if nan.any():
        gn = got[nan].astype(np.uint32)
        assert np.all((gn & 0x7C00) == 0x7C00) and np.all((gn & 0x03FF) != 0)
        assert np.array_equal(gn >> 15, patterns[nan].astype(np.uint32) >> 31)


def check_f16_decode(o: Oracle):
    """All 65536 binary16 patterns widen exactly, as numpy widens them."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got = o.f16_to_f32(h)
    want = h.astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def check_f16_codec_quick(o: Oracle):
    check_f16_rne(o, np.concatenate([special_f16_edges(), sampled_patterns(1 << 18, seed=21)]))
    check_f16_decode(o)


def check_f16_grad_and_param_out(o: Oracle, seed: int = 42):
    """fp16 gradients are widened exactly: the update equals the fp32 update
    of the widened gradient, bit for bit (both modes); an fp16 p_out is
    numpy's cast of the new fp32 param, including values beyond the fp16
    range (infinity) and below it (subnormals, zero)."""
    rng = np.random.default_rng(seed)
    n = 3001
    p0 = rng.standard_normal(n).astype(np.float32)
    p0[:8] = [70000.0, -70000.0, 65519.0, 1e-6, -3e-8, 0.0, 2.0 ** -20, 65504.0]
    g16 = (rng.standard_normal(n) * 1e-3).astype(np.float16)
    g16[:4] = np.array([6e-8, -6e-8, 1e-5, 60000.0], np.float16)  # subnormal, large
    g_wide = g16.astype(np.float32)
    for mode in (0, 1):
        hp = HParams(0.9, 0.95, 1e-8, 0.1, mode, 1)
        t16 = OracleTensor(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g16.copy(),
                           np.zeros(n, np.float16))
        t32 = OracleTensor(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g_wide.copy())
        s16, s32 = [0], [0]
        for _ in range(3):
            o.group_step([t16], hp, 1.6e-3, s16, 0.5)
            o.group_step([t32], hp, 1.6e-3, s32, 0.5)
            assert np.array_equal(t16.p.view(np.uint32), t32.p.view(np.uint32))
            assert np.array_equal(t16.v.view(np.uint32), t32.v.view(np.uint32))
            with np.errstate(over="ignore"):
                want = t32.p.astype(np.float16)
            assert np.array_equal(t16.p_out.view(np.uint16), want.view(np.uint16))


def check_f32_param_out(o: Oracle, seed: int = 45):
    """An fp32 param-out of fp32 params is the new param itself, bit for bit
    (the functor's cast to a float PARAM_OUT_T is the identity)."""
    rng = np.random.default_rng(seed)
    n = 1001
    p0 = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    for mode in (0, 1):
        hp = HParams(0.9, 0.95, 1e-8, 0.1, mode, 1)
        t = OracleTensor(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), g,
                         np.zeros(n, np.float32))
        st = [0]
        for _ in range(2):
            o.group_step([t], hp, 1.6e-3, st, 1.0)
            assert np.array_equal(t.p_out.view(np.uint32), t.p.view(np.uint32))


# ---------------------------------------------------------------------------
# 16-bit optimizer state (the state type T of the pages' functor = bf16/fp16)
# ---------------------------------------------------------------------------

def _library_round(x32: np.ndarray, kind: str) -> np.ndarray:
    """float32 -> bf16 bits (torch's CPU cast) or float16 (numpy's cast),
    both round to nearest even."""
    if kind == "f16":
        with np.errstate(over="ignore"):
            return np.ascontiguousarray(x32, np.float32).astype(np.float16)
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _library_widen(a: np.ndarray, kind: str) -> np.ndarray:
    if kind == "f16":
        return a.astype(np.float32)
    return (a.astype(np.uint32) << 16).view(np.float32)


def _bits16(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.float16 else a


def check_state16_update(o: Oracle, seed: int = 44):
    """16-bit state: p, m, v of one type T (bf16 or fp16) step as the pinned
    fp32 update of their widened values, with p, m and v then rounded to T by
    a library conversion (torch's float32 -> bfloat16, numpy's float32 ->
    float16); the param-out is the library cast of the new T param (an fp32
    param-out its exact widening).  Three steps, both modes, every gradient
    and param-out type; params include fp16 values next to its overflow
    threshold and subnormal second moments."""
    rng = np.random.default_rng(seed)
    n = 509
    for st in ("bf16", "f16"):
        p32 = rng.standard_normal(n).astype(np.float32)
        if st == "f16":
            p32[:4] = [65504.0, -65504.0, 65000.0, 6.1e-5]
        p0 = _library_round(p32, st)
        m0 = _library_round((rng.standard_normal(n) * 1e-3).astype(np.float32), st)
        v0 = _library_round((np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32), st)
        for g_kind in ("f32", "bf16", "f16"):
            g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
            g = g32 if g_kind == "f32" else _library_round(g32, g_kind)
            for out in (None, "f32", "bf16", "f16"):
                for mode in (0, 1):
                    hp = HParams(0.9, 0.95, 1e-8, 0.1, mode, 1)
                    p_out = None if out is None else np.zeros(
                        n, {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[out])
                    t16 = OracleTensor(p0.copy(), m0.copy(), v0.copy(), g, p_out)
                    t32 = OracleTensor(_library_widen(p0, st), _library_widen(m0, st),
                                       _library_widen(v0, st), g)
                    s16, s32 = [0], [0]
                    for _ in range(3):
                        o.group_step([t16], hp, 1.6e-3, s16, 0.5)
                        o.group_step([t32], hp, 1.6e-3, s32, 0.5)
                        for name in ("p", "m", "v"):
                            want = _library_round(getattr(t32, name), st)
                            assert np.array_equal(_bits16(getattr(t16, name)), _bits16(want)), \
                                (st, g_kind, out, mode, name)
                            setattr(t32, name, _library_widen(want, st))
                        if out is not None:
                            wide = _library_widen(t16.p, st)
                            if out == "f32":
                                assert np.array_equal(t16.p_out.view(np.uint32), wide.view(np.uint32))
                            else:
                                want_out = _library_round(wide, out)
                                assert np.array_equal(_bits16(t16.p_out), _bits16(want_out)), \
                                    (st, g_kind, out, mode, "p_out")


# ---------------------------------------------------------------------------
# Scaled 16-bit optimizer state
# ---------------------------------------------------------------------------

def _torch_state_dtype(state_dtype):
    import torch

    return torch.float16 if np.dtype(state_dtype) == np.float16 else torch.bfloat16


def _to_numpy_state(t, state_dtype) -> np.ndarray:
    import torch

    bits = t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return bits.view(np.float16) if np.dtype(state_dtype) == np.float16 else bits.copy()


def _from_numpy_state(a: np.ndarray, state_dtype):
    import torch

    bits = torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy())
    return bits.view(_torch_state_dtype(state_dtype))


def torch_apply_state_scale(x32: np.ndarray, state_dtype):
    """The per-tensor scaling that apex distributed_fused_adam.py defines in
    DistributedFusedAdam._apply_state_scale, and the copy into the state
    dtype T that follows it, restated from its mathematics in numpy float32
    (every operation one IEEE rounding):
        amax = max |X|                  (NaN if any element is NaN)
        L    = largest finite T / 2     (exact in float32 for bf16 and fp16)
        S    = amax / L
        r    = 1 / S if S > 0 else 0
        x    = T(X * r)                 (round to nearest even)
    The casts to T are library conversions: numpy's float16 cast, torch's
    CPU bfloat16 cast.  Returns (stored x as numpy bits, S)."""
    x = np.ascontiguousarray(x32, np.float32)
    fp16 = np.dtype(state_dtype) == np.float16
    big = np.float32(np.finfo(np.float16).max) if fp16 else np.float32(2.0 - 2.0 ** -7) * np.float32(2.0 ** 127)
    limit = big / np.float32(2.0)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        amax = np.max(np.abs(x))
        scale = np.float32(amax / limit)
        rscale = np.float32(np.float32(1.0) / scale) if scale > 0 else np.float32(0.0)
        y = (x * rscale).astype(np.float32)
        if fp16:
            stored = y.astype(np.float16)
        else:
            import torch

            stored = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return stored, np.float32(scale)


def torch_unscale(a: np.ndarray, scale, state_dtype) -> np.ndarray:
    """The pages' unscale: copy to float32, then multiply by the scale."""
    import torch

    t = _from_numpy_state(a, state_dtype).to(torch.float32)
    t.mul_(torch.tensor([float(scale)], dtype=torch.float32))
    return t.numpy().copy()


def _scaled_tensor(o: Oracle, rng, n: int, state_dtype, g, out_dtype):
    """Scaled state from p ~ N(0,1), m, v of mid-training size.  bf16 state
    takes m, v with magnitudes above 1: the pages' scale maps the largest
    magnitude to half of bf16's maximum (~1.7e38), so below ~0.5 the float
    reciprocal of the scale overflows (see the special cases)."""
    p0 = rng.standard_normal(n).astype(np.float32)
    if np.dtype(state_dtype) == np.float16:
        m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        v0 = (np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32)
    else:
        m0 = (rng.standard_normal(n) * 4.0).astype(np.float32)
        v0 = (np.abs(rng.standard_normal(n)) * 4.0 + 1.0).astype(np.float32)
    parts = [torch_apply_state_scale(x, state_dtype) for x in (p0, m0, v0)]
    scales = np.array([sc for _, sc in parts], np.float32)
    p_out = None if out_dtype is None else np.zeros(n, out_dtype)
    return OracleTensor(parts[0][0], parts[1][0], parts[2][0], g, p_out, None, scales)


def check_scaled_state(o: Oracle, seed: int = 43):
    """Scaled state, both state types: (1) the oracle's scaling of a float
    buffer equals the pages' torch sequence bit for bit; (2) three steps equal
    [torch unscale -> the pinned fp32 update -> torch casts for p_out ->
    torch rescale], bit for bit in p, m, v, the three scales and p_out;
    (3) the largest stored magnitude is half the type's maximum, rounded;
    (4) dequantised values are within the type's relative precision of the
    float32 values they came from."""
    rng = np.random.default_rng(seed)
    n = 1537
    for state_dtype, out_dtype, g_dtype in ((np.uint16, np.uint16, np.float32),
                                            (np.float16, np.float16, np.uint16),
                                            (np.uint16, np.float16, np.float16),
                                            (np.float16, None, np.float32)):
        limit = o.scaled_state_limit(state_dtype)
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
        got, sc = o.scale_state(x, state_dtype)
        want, wsc = torch_apply_state_scale(x, state_dtype)
        assert sc == wsc and np.array_equal(got.view(np.uint16), want.view(np.uint16))
        g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        g = g32 if g_dtype == np.float32 else (
            g32.astype(np.float16) if g_dtype == np.float16 else torch_bf16_bits(g32))
        for mode in (0, 1):
            hp = HParams(0.9, 0.95, 1e-8, 0.1, mode, 1)
            t = _scaled_tensor(o, rng, n, state_dtype, g.copy(), out_dtype)
            ref = OracleTensor(t.p.copy(), t.m.copy(), t.v.copy(), g.copy(), None, None, t.scales.copy())
            st, sr = [0], [0]
            for _ in range(3):
                o.group_step([t], hp, 1.6e-3, st, 1.0)
                # reference: unscale, fp32 update, casts, rescale
                f = OracleTensor(torch_unscale(ref.p, ref.scales[0], state_dtype),
                                 torch_unscale(ref.m, ref.scales[1], state_dtype),
                                 torch_unscale(ref.v, ref.scales[2], state_dtype), g.copy())
                o.group_step([f], hp, 1.6e-3, sr, 1.0)
                if out_dtype is not None:
                    import torch

                    cast = torch.from_numpy(f.p.copy()).to(_torch_state_dtype(out_dtype))
                    assert np.array_equal(t.p_out.view(np.uint16),
                                          _to_numpy_state(cast, out_dtype).view(np.uint16))
                for k, (name, arr) in enumerate((("p", f.p), ("m", f.m), ("v", f.v))):
                    stored, scale = torch_apply_state_scale(arr, state_dtype)
                    assert scale == t.scales[k], (name, scale, t.scales[k])
                    assert np.array_equal(getattr(t, name).view(np.uint16), stored.view(np.uint16)), name
                    setattr(ref, name, stored)
                    ref.scales[k] = scale
                    # largest stored magnitude sits at the limit, within rounding
                    dec = torch_unscale(stored, 1.0, state_dtype).astype(np.float64)
                    top = np.max(np.abs(dec))
                    rel = 2.0 ** -8 if state_dtype == np.uint16 else 2.0 ** -11
                    assert abs(top - float(limit)) <= 2 * rel * float(limit), (name, top, limit)
                    # dequantised values track the float values
                    back = dec * float(scale)
                    tol = rel * np.abs(arr.astype(np.float64)) + float(scale) * 2.0 ** -24 + 1e-45
                    if state_dtype == np.float16:  # binary16 subnormals: absolute spacing
                        tol = tol + float(scale) * 2.0 ** -25
                    assert np.all(np.abs(back - arr) <= tol * 1.01), name


def check_scaled_state_special_cases(o: Oracle):
    """Closed forms: an all-zero buffer gets scale 0 and stores zeros (and
    unscales to zeros); a buffer whose largest magnitude is the limit times
    2^k gets scale 2^k exactly and stores RNE(x / 2^k); a NaN makes the scale
    NaN and every stored finite value a zero; an infinity makes the scale
    infinite, the infinity NaN, and every finite value a zero."""
    for state_dtype in (np.uint16, np.float16):
        limit = float(o.scaled_state_limit(state_dtype))
        z, sc = o.scale_state(np.zeros(17, np.float32), state_dtype)
        assert sc == 0.0 and not np.any(z.view(np.uint16) & 0x7FFF)
        rng = np.random.default_rng(44)
        for k in (-30, -3, 0):
            x = (rng.uniform(-1, 1, 257) * limit * 2.0 ** k).astype(np.float32)
            x[100] = np.float32(-limit * 2.0 ** k)
            got, sc = o.scale_state(x, state_dtype)
            assert sc == np.float32(2.0 ** k), (k, sc)
            want = (x / np.float32(2.0 ** k)).astype(np.float32)
            if state_dtype == np.float16:
                assert np.array_equal(got.view(np.uint16), want.astype(np.float16).view(np.uint16))
            else:
                assert np.array_equal(got, torch_bf16_bits(want))
        # bf16 range: a largest magnitude below ~0.5 gives a subnormal scale
        # whose float reciprocal overflows, so finite values store as +-inf
        # (the torch sequence does the same)
        if state_dtype == np.uint16:
            x = np.array([1e-3, -2e-4, 0.0, 0.25], np.float32)
            got, sc = o.scale_state(x, state_dtype)
            want, wsc = torch_apply_state_scale(x, state_dtype)
            assert sc == wsc and 0 < sc < np.finfo(np.float32).tiny
            # 0 * inf is NaN: compare NaN as NaN (payloads differ)
            assert list(got[[0, 1, 3]]) == list(want[[0, 1, 3]]) == [0x7F80, 0xFF80, 0x7F80]
            assert (int(got[2]) & 0x7FFF) > 0x7F80 and (int(want[2]) & 0x7FFF) > 0x7F80
        for bad in (np.nan, np.inf):
            x = np.array([1.0, -2.0, bad, 0.5], np.float32)
            got, sc = o.scale_state(x, state_dtype)
            want_scale_nan = bool(np.isnan(bad))
            assert np.isnan(sc) if want_scale_nan else sc == np.inf
            bits = got.view(np.uint16).astype(np.uint32)
            fin = np.isfinite(x)
            assert np.all((bits[fin] & 0x7FFF) == 0)  # finite * 0 = signed zero
            dec = torch_unscale(got[~fin], 1.0, state_dtype)
            assert np.all(np.isnan(dec))


QUICK_CHECKS = (
    "check_bias_corrections_quick",
    "check_first_step_adamw",
    "check_first_step_l2",
    "check_first_step_no_bias_correction",
    "check_constant_gradient_closed_form",
    "check_zero_gradient",
    "check_random_runs_vs_shadow_quick",
    "check_against_torch_optim",
    "check_bf16_rne_quick",
    "check_remainder_codec_quick",
    "check_param_out_and_remainder_update",
    "check_noop_and_counter",
    "check_grad_sumsq",
    "check_clip_grad_scale",
    "check_f16_codec_quick",
    "check_f16_grad_and_param_out",
    "check_scaled_state",
    "check_scaled_state_special_cases",
    "check_f32_param_out",
    "check_state16_update",
)


def check_bias_corrections_quick(o: Oracle):
    check_bias_corrections(o, betas=(0.9, 0.999), steps=tuple(range(1, 40)) + (1000, 2**31 - 1))


def check_random_runs_vs_shadow_quick(o: Oracle):
    check_random_runs_vs_shadow(o, trials=12)


def sampled_patterns(count: int = 1 << 20, seed: int = 20) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.concatenate([special_f32_patterns(),
                           rng.integers(0, 2**32, size=count, dtype=np.uint64).astype(np.uint32)])


def check_bf16_rne_quick(o: Oracle):
    check_bf16_rne(o, sampled_patterns())


def check_remainder_codec_quick(o: Oracle):
    check_remainder_codec(o, sampled_patterns())


def run_quick(o: Oracle, stop_at_first: bool = False):
    """Runs the quick checks; returns the list of (name, error) failures."""
    failures = []
    for name in QUICK_CHECKS:
        try:
            globals()[name](o)
        except (AssertionError, FloatingPointError, ValueError, OverflowError) as e:
            failures.append((name, repr(e)[:200]))
            if stop_at_first:
                break
    return failures
