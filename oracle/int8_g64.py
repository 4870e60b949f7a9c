"""INT8 group-64 cache cells (oracle; test infrastructure only).

Format (strata PR #2698, section "What it does"): each K or V head vector is
stored as int8 codes plus one FP16 scale for every 64 consecutive values, the
scale being the group's max-abs divided by 127.  Codes round half to even
(strata PR #120, section "Tests", which names ties-to-even for the INT8 rules).

Readings where the pages are silent:
  * the groups are 64 consecutive values along head_dim of one (token, head) vector;
  * codes are made by dividing by the binary32 scale absmax/127 (the FP16 value
    is what is stored and what dequantisation multiplies by);
  * codes are clamped to [-127, 127];
  * an all-zero group stores scale +0 and codes 0.
"""
from __future__ import annotations

import numpy as np

from .numerics import F32, to_f16

GROUP = 64
QMAX = 127


def code_bytes(head_dim: int) -> int:
    return head_dim


def n_scales(head_dim: int) -> int:
    return head_dim // GROUP


def encode(x: np.ndarray):
    """x: float32 [..., D] (D % 64 == 0) -> (codes int8 [..., D], scales float16 [..., D/64])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % GROUP:
        raise ValueError("head_dim must be a multiple of 64")
    g = x.reshape(*x.shape[:-1], D // GROUP, GROUP)
    absmax = np.max(np.abs(g), axis=-1)                       # exact
    nonzero = absmax > 0
    scale = absmax / F32(QMAX)                                # binary32, correctly rounded
    divisor = np.where(nonzero, scale, F32(1))[..., None]
    q = np.rint(g / divisor)                                  # correctly rounded divide, then half-to-even
    q = np.clip(q, -QMAX, QMAX)
    codes = np.where(nonzero[..., None], q, F32(0)).astype(np.int8).reshape(x.shape)
    scales = to_f16(np.where(nonzero, scale, F32(0)))
    return codes, scales


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes int8 [..., D], scales float16 [..., D/64]) -> float32 [..., D]; code * scale is exact in binary32."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    c = codes.astype(np.float32).reshape(*codes.shape[:-1], D // GROUP, GROUP)
    s = np.asarray(scales).astype(np.float32)[..., None]
    return (c * s).reshape(codes.shape)
