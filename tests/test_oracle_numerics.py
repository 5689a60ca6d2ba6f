"""Pins for oracle.numerics: exact widening of stored fp32/fp16/bf16 values.

Expected values are textbook IEEE-754 / bfloat16 encodings, not recomputed by
the oracle's own route.
"""
import numpy as np
import pytest

from oracle.numerics import to_f64, F32, F16, BF16


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
    (0x3555, 0.333251953125), (0x8000, -0.0), (0x0400, 2.0 ** -14),
])
def test_f16_encodings(bits, value):
    got = to_f64(np.array([bits], dtype=np.uint16), F16)[0]
    assert got == value and np.signbit(got) == np.signbit(value)


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133),
    (0x7F7F, 3.3895313892515355e38), (0x3E80, 0.25),
])
def test_bf16_encodings(bits, value):
    assert to_f64(np.array([bits], dtype=np.uint16), BF16)[0] == value


@pytest.mark.parametrize("bits,value", [
    (0x3F800000, 1.0), (0x40490FDB, 3.1415927410125732), (0x00000001, 2.0 ** -149),
])
def test_f32_encodings(bits, value):
    assert to_f64(np.array([bits], dtype=np.uint32), F32)[0] == value


def test_bf16_nan_inf():
    v = to_f64(np.array([0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16), BF16)
    assert v[0] == np.inf and v[1] == -np.inf and np.isnan(v[2])


def test_wrong_carrier_rejected():
    with pytest.raises(TypeError):
        to_f64(np.zeros(2, dtype=np.uint32), F16)
