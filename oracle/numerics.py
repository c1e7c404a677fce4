"""Exact decoding of stored element formats to float64 (oracle side)."""
import numpy as np

BF16 = "bf16"
F32 = "f32"
F64 = "f64"   # float64 intermediates of the oracle itself, taken as they are


def decode(a, dtype: str) -> np.ndarray:
    """Stored tensor -> float64, exactly.

    bf16 tensors arrive as their uint16 bit patterns; a bf16 value is the
    float32 whose upper 16 bits are those bits and whose lower 16 bits are 0.
    """
    a = np.asarray(a)
    if dtype == BF16:
        bits = a.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == F32:
        return a.astype(np.float32).astype(np.float64)
    if dtype == F64:
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
