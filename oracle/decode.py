"""Exact decoding of stored tensors to float64 (oracle; test infrastructure only)."""

import numpy as np


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Return the float64 value of every stored element.

    ``dtype`` is "f32" (IEEE single) or "bf16" (raw 16-bit bfloat16 patterns
    held in uint16). A bfloat16 value is the float32 whose upper 16 bits are
    the pattern and whose lower 16 bits are zero, so widening is exact.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError("unknown storage type %r" % (dtype,))
