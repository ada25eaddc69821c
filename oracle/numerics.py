"""Exact widening of stored input values to float64 (oracle; test infrastructure only)."""
import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64, exactly.

    A bfloat16 value is the upper half of the float32 with the same bits, so
    shifting the pattern into the high half of a 32-bit word gives the float32,
    which widens to float64 without rounding.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input (bf16 bits or fp32 values) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
