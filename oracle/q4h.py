"""Walsh-Hadamard-rotated q4_0 cache cells (the V side of k8v4; oracle, test infrastructure only).

Method (strata PR #120, sections "What" and "How"; strata PR #2698, section
"Not in this PR"): a V head vector of 256 values is rotated by the orthonormal
Walsh-Hadamard transform (FWHT-256), then quantised as q4_0 -- blocks of 32
values, one FP16 ``d`` per block equal to the block's signed max-abs value
divided by -8, and 4-bit codes ``clamp(round(z/d) + 8, 0, 15)``.  Attention
accumulates in the rotated basis and rotates its output back.

Readings where the pages are silent:
  * H = H_256 / 16 with H_256 the Sylvester-ordered Hadamard matrix
    (entry (i, j) is (-1)^popcount(i & j)), no random sign flips;
  * binary32 evaluation order of the transform: butterfly stages of span
    1, 2, 4, ..., 128, each pair (a, b) -> (a + b, a - b), then one exact
    scaling by 1/16;
  * "signed max-abs" is the first value in block order whose magnitude is largest;
  * codes divide by the binary32 d = m / -8 (exact) and round half to even;
  * an all-zero block stores d = +0 and codes 8;
  * byte j of a head-cell holds code 2j in its low nibble and code 2j+1 in its high nibble.
"""
from __future__ import annotations

import numpy as np

from .numerics import F32, to_f16

DIM = 256
BLOCK = 32


def code_bytes(head_dim: int) -> int:
    return head_dim // 2


def n_scales(head_dim: int) -> int:
    return head_dim // BLOCK


def fwht256(y: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis (length 256), binary32.

    It is its own inverse: H is symmetric and H @ H = I."""
    y = np.array(y, dtype=np.float32, copy=True)
    if y.shape[-1] != DIM:
        raise ValueError("FWHT-256 needs head_dim 256")
    lead = y.shape[:-1]
    h = 1
    while h < DIM:
        pairs = y.reshape(*lead, DIM // (2 * h), 2, h)   # element i pairs with i + h where bit h of i is 0
        a = pairs[..., 0, :].copy()
        b = pairs[..., 1, :].copy()
        pairs[..., 0, :] = a + b
        pairs[..., 1, :] = a - b
        h *= 2
    return y * F32(1.0 / 16.0)


def q4_0_encode(z: np.ndarray):
    """z: float32 [..., D] (D % 32 == 0) -> (packed uint8 [..., D/2], d float16 [..., D/32])."""
    z = np.asarray(z, dtype=np.float32)
    D = z.shape[-1]
    blk = z.reshape(*z.shape[:-1], D // BLOCK, BLOCK)
    first = np.argmax(np.abs(blk), axis=-1)                   # first index of the largest magnitude
    m = np.take_along_axis(blk, first[..., None], axis=-1)[..., 0]
    nonzero = m != 0
    d = m / F32(-8)                                           # exact: a power-of-two divide
    divisor = np.where(nonzero, d, F32(1))[..., None]
    q = np.rint(blk / divisor) + F32(8)
    q = np.clip(q, 0, 15)
    codes = np.where(nonzero[..., None], q, F32(8)).astype(np.uint8).reshape(z.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, to_f16(np.where(nonzero, d, F32(0)))


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0x0F)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def q4_0_decode(packed: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Dequantise in the rotated basis: (code - 8) * d, exact in binary32."""
    codes = unpack_nibbles(packed).astype(np.float32) - F32(8)
    D = codes.shape[-1]
    blk = codes.reshape(*codes.shape[:-1], D // BLOCK, BLOCK)
    return (blk * np.asarray(d).astype(np.float32)[..., None]).reshape(codes.shape)


def encode(v: np.ndarray):
    """V head vectors float32 [..., 256] -> q4_0 cells of their Hadamard rotation."""
    return q4_0_encode(fwht256(v))


def decode_rotated(packed, d) -> np.ndarray:
    """The stored values, still in the rotated basis (what the cache holds), binary32."""
    return q4_0_decode(packed, d)


def decode(packed, d) -> np.ndarray:
    """The stored values rotated back to the original basis, in fp64 (H applied exactly)."""
    y = q4_0_decode(packed, d).astype(np.float64)
    return hadamard_f64(y)


def hadamard_f64(y: np.ndarray) -> np.ndarray:
    """Apply H = H_256/16 in fp64 by its definition, entry (i, j) = (-1)^popcount(i & j) / 16."""
    i = np.arange(DIM)
    parity = np.zeros((DIM, DIM), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    H = np.where(parity == 1, -1.0, 1.0) / 16.0
    return np.asarray(y, dtype=np.float64) @ H.T
