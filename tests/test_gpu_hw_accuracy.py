"""The hardware facts the scaled-state maxima pass relies on, measured on the
device the tests run on over every float input (tests/hw/hw_accuracy.hip):
the fp32 square root and reciprocal instructions are within 2^-23 (one
ulp, half the 2^-22 the pass's error bound assumes) of the exact values for
normal inputs (square root: every normal input; reciprocal: inputs below
2^126, whose reciprocal is normal); a reciprocal of a subnormal input is
+inf or accurate; sqrt(0) = 0 and rcp(+inf) = 0.  And the one the one-pass
scaled kernel's stores rely on: the float -> bf16 conversion instruction
rounds every float to nearest even, NaN payloads as the integer form."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libhw_accuracy.so")


@pytest.fixture(scope="module")
def measured():
    from gpu_helpers import torch_mod

    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(LIB), "tests/hw/libhw_accuracy.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    sq = np.zeros(255, np.float64)
    rc = np.zeros(255, np.float64)
    loose = ctypes.c_uint32(0)
    sp = np.zeros(4, np.float32)
    dp = ctypes.POINTER(ctypes.c_double)
    status = lib.hw_accuracy(sq.ctypes.data_as(dp), rc.ctypes.data_as(dp), ctypes.byref(loose),
                             sp.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    assert status == 0
    return sq, rc, loose.value, sp


def test_square_root_within_one_ulp_for_normal_inputs(measured):
    sq = measured[0]
    worst = sq[1:255].max()
    print(f"sqrt: largest relative error over normal inputs {worst / 2.0 ** -23:.4f} x 2^-23")
    assert worst < 2.0 ** -23


def test_reciprocal_within_one_ulp_where_the_result_is_normal(measured):
    rc, loose = measured[1], measured[2]
    worst = rc[1:253].max()  # inputs in [2^-126, 2^126)
    print(f"rcp: largest relative error over [2^-126, 2^126) {worst / 2.0 ** -23:.4f} x 2^-23")
    assert worst < 2.0 ** -23
    assert loose == 0, "a finite reciprocal of an input below 2^126 off by more than 2^-23"


def test_special_values(measured):
    sp = measured[3]
    assert sp[0] == 0.0 and not np.signbit(sp[0])
    assert sp[1] == 0.0
    assert np.isinf(sp[2]) and sp[2] > 0
    assert np.isinf(sp[3]) and sp[3] > 0


def test_bf16_conversion_instruction_rounds_to_nearest_even():
    from gpu_helpers import torch_mod

    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(LIB), "tests/hw/libhw_accuracy.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    mismatches, first = ctypes.c_uint64(0), ctypes.c_uint32(0)
    assert lib.bf16_conversion(ctypes.byref(mismatches), ctypes.byref(first)) == 0
    assert mismatches.value == 0, f"{mismatches.value} floats differ, first {first.value:#010x}"
