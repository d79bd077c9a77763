"""The error bound of the scaled-state maxima pass, checked on the CPU.

The maxima pass computes each param with the hardware square root and
reciprocal, bounds the distance to the exact IEEE param by a per-wave E, and
recomputes exactly only the elements with |p~| >= max|p~| - 2.5 E.  These
tests restate that computation in numpy float32 (correctly rounded, denormals
kept) with the hardware results replaced by the correctly rounded value moved
by -1, 0 or +1 ulp at random (the measured hardware error is below 0.78 ulp,
tests/test_gpu_hw_accuracy.py), on 256-element groups (one wave's lanes x 4)
drawn to stress the bound: ties, cancellation between the Adam term and the
decay, magnitudes over the whole float range, subnormal moments, extreme
hyperparameters.  They check that every element lies within E of its exact
value and that the selected elements hold the exact maximum."""
import numpy as np
import pytest

f = np.float32
N = 256


def _nudge(x, k):
    out = x.copy()
    up, dn = k > 0, k < 0
    out[up] = np.nextafter(x[up], f(np.inf))
    out[dn] = np.nextafter(x[dn], f(-np.inf))
    return np.where(np.isfinite(x) & (x != 0), out, x)


def _chains(p, mh, vh, lr, wd, eps, mode, ks, kr):
    """Exact param and the approximate chain's q~, u~, t~, p~."""
    with np.errstate(all="ignore"):
        q = f(mh / f(np.sqrt(vh) + eps))
        u = f(q + f(wd * p)) if mode == 1 else q
        pe = f(p - f(lr * u))
        sa = _nudge(np.sqrt(vh), ks)
        # the hardware flushes subnormal inputs of either sign: sqrt to a
        # zero of the input's sign, rcp to +inf
        sa = np.where((vh != 0) & (np.abs(vh) < f(2.0 ** -126)), np.copysign(f(0.0), vh), sa)
        da = f(sa + eps)
        ra = np.where(da < f(2.0 ** -126), f(np.inf), _nudge(f(f(1.0) / da), kr))
        qa = f(mh * ra)
        ua = f(qa + f(wd * p)) if mode == 1 else qa
        ta = f(lr * ua)
        pa = f(p - ta)
    return pe, qa, ua, ta, pa


def _abs_bits(x):
    return x.view(np.uint32) & np.uint32(0x7FFFFFFF)


def _group(rng, kind):
    mode = int(rng.integers(2))
    lr = f(rng.choice([1e-3, 1.6e-3, 0.5, 3.0, 1e-30, 1e20, 0.0, -1e-3]))
    wd = f(rng.choice([0.0, 0.01, 0.1, 1.0, 100.0]))
    eps = f(rng.choice([0.0, 1e-8, 1e-3, 1.0, 1e-40, 1e30]))
    if kind == "typical":
        p = f(rng.standard_normal(N)); mh = f(rng.standard_normal(N) * 1e-3)
        vh = f(np.abs(rng.standard_normal(N)) * 1e-6)
    elif kind == "ties":
        p = np.full(N, f(rng.standard_normal()), f); mh = np.full(N, f(rng.standard_normal()), f)
        vh = np.full(N, f(abs(rng.standard_normal())), f)
        p[rng.integers(N, size=5)] = np.nextafter(p[0], f(np.inf))
    elif kind == "cancellation":  # the Adam term close to minus the decay
        p = f(rng.standard_normal(N)); vh = f(np.abs(rng.standard_normal(N)))
        mh = f(-wd * p * (np.sqrt(vh) + eps) * (1 + rng.standard_normal(N) * 1e-6))
    elif kind == "wide":
        p = f(rng.standard_normal(N) * 10.0 ** rng.integers(-40, 38, N))
        mh = f(rng.standard_normal(N) * 10.0 ** rng.integers(-40, 30, N))
        vh = f(np.abs(rng.standard_normal(N)) * 10.0 ** rng.integers(-37, 38, N) + 1.2e-38)
    elif kind == "update_dominated":
        p = f(rng.standard_normal(N) * 1e-6); mh = f(rng.standard_normal(N))
        vh = f(mh.astype(np.float64) ** 2 * (1 + rng.random(N) * 1e-5))
    else:  # tiny: subnormal params and first moments, v_hat zero or just normal
        p = f(rng.standard_normal(N) * 1e-38); mh = f(rng.standard_normal(N) * 1e-42)
        vh = f(np.abs(rng.standard_normal(N)) * 1e-37 + 1.2e-38)
        vh[rng.random(N) < 0.2] = 0
    return p, mh, vh, lr, wd, eps, mode


def _bound(qa, ta, pa, lr):
    """E as the kernel forms it (from the maxima of the group)."""
    alr = f(abs(lr))
    with np.errstate(all="ignore"):
        return f(f(f(f(f(2.0 ** -19) * alr) * np.max(np.abs(qa))) + f(f(2.0 ** -21) * np.max(np.abs(ta))))
                 + f(f(f(2.0 ** -22) * f(_abs_bits(pa).max().view(np.float32)))
                     + f(f(2.0 ** -140) * f(alr + f(1.0)))))


def _valid(eps, lr, vh, qa, ua, ta, pa):
    """The kernel's conditions for using the bound (else: every element exact)."""
    return (eps >= 0 and eps < 2.0 ** 125 and abs(lr) < 2.0 ** 126
            and not np.any((vh != 0) & (np.abs(vh) < f(2.0 ** -126)))
            and _abs_bits(pa).max() < 0x7E800000
            and np.nanmax(np.abs(qa)) < 2.0 ** 126 and np.nanmax(np.abs(ua)) < 2.0 ** 126
            and np.nanmax(np.abs(ta)) < 2.0 ** 126)


KINDS = ["typical", "ties", "cancellation", "wide", "update_dominated", "tiny"]


@pytest.mark.parametrize("kind", KINDS)
def test_bound_holds_and_the_exact_maximum_is_kept(kind):
    rng = np.random.default_rng(KINDS.index(kind) + 500)
    used = 0
    for _ in range(2000):
        p, mh, vh, lr, wd, eps, mode = _group(rng, kind)
        ks, kr = rng.integers(-1, 2, N), rng.integers(-1, 2, N)
        pe, qa, ua, ta, pa = _chains(p, mh, vh, lr, wd, eps, mode, ks, kr)
        if not _valid(eps, lr, vh, qa, ua, ta, pa):
            continue
        used += 1
        E = _bound(qa, ta, pa, lr)
        err = np.abs(pa.astype(np.float64) - pe.astype(np.float64))
        assert np.all(err <= E), (kind, mode, lr, wd, eps, err.max(), E)
        top = f(_abs_bits(pa).max().view(np.float32))
        cut = f(top - f(f(2.5) * E))
        chosen = np.abs(pa) >= cut
        assert _abs_bits(pe[chosen]).max() == _abs_bits(pe).max(), (kind, mode)
    assert used > 100, f"too few groups inside the bound's assumptions: {used}"


def test_typical_groups_recompute_few_elements():
    """On a typical optimizer state the cut keeps a handful of a wave's
    elements, so the exact recompute is rare."""
    rng = np.random.default_rng(7)
    counts = []
    for _ in range(300):
        p = f(rng.standard_normal(N)); mh = f(rng.standard_normal(N) * 1e-3)
        vh = f(np.abs(rng.standard_normal(N)) * 1e-6)
        pe, qa, ua, ta, pa = _chains(p, mh, vh, f(1.6e-3), f(0.1), f(1e-8), 1,
                                     rng.integers(-1, 2, N), rng.integers(-1, 2, N))
        E = _bound(qa, ta, pa, f(1.6e-3))
        cut = f(f(_abs_bits(pa).max().view(np.float32)) - f(f(2.5) * E))
        counts.append(int((np.abs(pa) >= cut).sum()))
    assert np.mean(counts) < 1.5 and max(counts) <= 4


def test_subnormal_second_moment_takes_the_exact_path():
    """A subnormal v_hat (the hardware square root flushes it) puts its whole
    wave outside the bound's assumptions."""
    rng = np.random.default_rng(9)
    p = f(rng.standard_normal(N)); mh = f(rng.standard_normal(N) * 1e-3)
    vh = f(np.abs(rng.standard_normal(N)) * 1e-6)
    vh[17] = f(1e-40)
    pe, qa, ua, ta, pa = _chains(p, mh, vh, f(1.6e-3), f(0.1), f(1e-8), 1, np.zeros(N, int), np.zeros(N, int))
    assert not _valid(f(1e-8), f(1.6e-3), vh, qa, ua, ta, pa)
    assert _valid(f(1e-8), f(1.6e-3), np.where(vh < 1e-38, f(0.0), vh), qa, ua, ta, pa)


def test_negative_second_moment_takes_the_exact_path():
    """A negative v_hat (a negative stored v or scale): the exact root is NaN.
    The hardware root of a negative subnormal is the flushed -0, so the
    approximate param comes out finite where the exact one is NaN; of a
    negative normal it is NaN, as the exact one.  Both put the wave outside
    the bound's assumptions, so every element is recomputed exactly and the
    NaN reaches the maximum."""
    rng = np.random.default_rng(11)
    p = f(rng.standard_normal(N)); mh = f(rng.standard_normal(N) * 1e-3)
    vh = f(np.abs(rng.standard_normal(N)) * 1e-6)
    for bad in (f(-1e-40), f(-2.0 ** -149), f(-1e-6), f(-3.0)):
        v = vh.copy()
        v[33] = bad
        pe, qa, ua, ta, pa = _chains(p, mh, v, f(1.6e-3), f(0.1), f(1e-8), 1, np.zeros(N, int),
                                     np.zeros(N, int))
        assert np.isnan(pe[33])
        if bad > f(-2.0 ** -126):
            assert np.isfinite(pa[33])  # the hazard: the approximate chain misses the NaN
        else:
            assert np.isnan(pa[33])
        assert not _valid(f(1e-8), f(1.6e-3), v, qa, ua, ta, pa)
