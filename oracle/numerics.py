"""Binary32 primitives shared by the oracle's encoders (oracle-internal; test infrastructure).

numpy applies one IEEE-754 rounding per ufunc call on float32 arrays and never
fuses a multiply into an add, so writing each step of an encoder as its own
numpy expression reproduces the binary32 arithmetic the encoders specify.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32; exact, a bf16 is the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f16(x) -> np.ndarray:
    """binary32 -> binary16, round to nearest, ties to even, subnormals kept, overflow to inf."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def tree_sum(x) -> np.ndarray:
    """Sum along the last axis (length a power of two) in a fixed order: add the upper half
    onto the lower half, elementwise, until one value is left.  Each add is one binary32 rounding."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError("tree_sum needs a power-of-two length")
    while n > 1:
        h = n // 2
        y[..., :h] = y[..., :h] + y[..., h:n]
        n = h
    return y[..., 0]
