"""Exact conversion of stored KV/query values to float64 (oracle, test-only).

The pages fix no precision ([P2 §1.1] states only the formula).  The stored
element types are fp32, IEEE fp16 and bfloat16; every one of them converts to
float64 exactly, so the oracle's attention runs on the exact stored values.

Values are carried as raw bit patterns (``uint32`` for fp32, ``uint16`` for
fp16/bf16) so that no float round-trip can disturb bitwise comparisons of KV
bytes.  bfloat16 is the upper half of an IEEE binary32 pattern, so its exact
widening is a 16-bit left shift followed by a binary32 reinterpretation.
"""
import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"
DTYPES = (F32, F16, BF16)

_BITS = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}
_ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}


def bits_dtype(dtype):
    """Unsigned integer type that carries one stored element of ``dtype``."""
    return _BITS[dtype]


def elem_bytes(dtype):
    return _ELEM_BYTES[dtype]


def to_f64(bits, dtype):
    """Widen an array of stored bit patterns to float64 without rounding."""
    bits = np.asarray(bits)
    if bits.dtype != _BITS[dtype]:
        raise TypeError(f"{dtype} values must be carried as {_BITS[dtype].__name__}")
    if dtype == F32:
        return bits.view(np.float32).astype(np.float64)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)
