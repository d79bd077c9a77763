"""The oracle against its pins (CPU only).  See tests/pins.py for what each
check compares with."""
import os

import numpy as np
import pytest

import pins


def _golden_steps(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "empty_group_steps.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals["populated"], vals["empty"]


def test_bias_corrections_exact(oracle_default):
    pins.check_bias_corrections(oracle_default)


def test_first_step_adamw_closed_form(oracle_default):
    pins.check_first_step_adamw(oracle_default)


def test_first_step_l2_closed_form(oracle_default):
    pins.check_first_step_l2(oracle_default)


def test_first_step_without_bias_correction(oracle_default):
    pins.check_first_step_no_bias_correction(oracle_default)


def test_constant_gradient_closed_form(oracle_default):
    pins.check_constant_gradient_closed_form(oracle_default)
    pins.check_constant_gradient_closed_form(oracle_default, steps=100)


def test_zero_gradient_recurrence_bitwise(oracle_default):
    pins.check_zero_gradient(oracle_default)


def test_random_runs_vs_float64_shadow(oracle_default):
    pins.check_random_runs_vs_shadow(oracle_default)


def test_against_torch_optim_float64(oracle_default):
    pins.check_against_torch_optim(oracle_default)


def test_param_out_and_remainder_update(oracle_default):
    pins.check_param_out_and_remainder_update(oracle_default)


def test_noop_and_counter(oracle_default):
    pins.check_noop_and_counter(oracle_default)


def test_empty_group_counter_matches_pages(oracle_default, golden_dir):
    pins.check_empty_group_counter(oracle_default, _golden_steps(golden_dir))


def test_grad_sumsq_is_the_correctly_rounded_sum(oracle_default):
    pins.check_grad_sumsq(oracle_default)


def test_clip_grad_scale_matches_torch_clip(oracle_default):
    pins.check_clip_grad_scale(oracle_default)


def test_f16_cast_edges_and_decode(oracle_default):
    pins.check_f16_rne(oracle_default, pins.special_f16_edges())
    pins.check_f16_decode(oracle_default)


def test_f16_gradients_and_param_out(oracle_default):
    pins.check_f16_grad_and_param_out(oracle_default)


def test_scaled_state_matches_the_pages_torch_sequence(oracle_default):
    pins.check_scaled_state(oracle_default)


def test_f32_param_out_is_the_new_param(oracle_default):
    pins.check_f32_param_out(oracle_default)


def test_state16_update_is_the_rounded_fp32_update(oracle_default):
    pins.check_state16_update(oracle_default)


def test_scaled_state_special_cases(oracle_default):
    pins.check_scaled_state_special_cases(oracle_default)


def test_host_counter_overflow_wraps_like_int32(oracle_default):
    from oracle import HParams

    step = [2**31 - 1]
    oracle_default.group_step([], HParams(), 1e-3, step, 1.0, noop=0)
    assert step == [-(2**31)]


def test_bf16_rne_special_patterns(oracle_default):
    pins.check_bf16_rne(oracle_default, pins.special_f32_patterns())


def test_remainder_codec_special_patterns(oracle_default):
    pins.check_remainder_codec(oracle_default, pins.special_f32_patterns())


CHUNK = 1 << 24


def _over_all_patterns(fn):
    """Runs fn(patterns) over all 2^32 float32 bit patterns, in chunks, on a
    few threads (the C calls and numpy release the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(start):
        fn(np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32))

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(0, 1 << 32, CHUNK)))


@pytest.mark.slow
def test_bf16_rne_exhaustive(oracle_default):
    """All 2^32 float32 bit patterns against torch's cast."""
    _over_all_patterns(lambda pats: pins.check_bf16_rne(oracle_default, pats))


@pytest.mark.slow
def test_f16_rne_exhaustive(oracle_default):
    """All 2^32 float32 bit patterns against numpy's float32 -> float16 cast."""
    _over_all_patterns(lambda pats: pins.check_f16_rne(oracle_default, pats))


@pytest.mark.slow
def test_remainder_round_trip_exhaustive(oracle_default):
    """All 2^32 float32 bit patterns: exact round trip and the layout split;
    the nearest-value property on every 97th pattern (all exponents, signs)."""
    o = oracle_default

    def one(pats):
        hi, lo = o.rem_encode(pats.view(np.float32))
        assert np.array_equal(o.rem_decode(hi, lo).view(np.uint32), pats)
        assert np.array_equal(lo, pats.view(np.int16).reshape(-1, 2)[:, 0])
        pins.check_remainder_codec(o, pats[::97].copy())

    _over_all_patterns(one)
