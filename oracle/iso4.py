"""ISO4 (IsoQuant 4-bit) cache cells (oracle; test infrastructure only).

FreeToken PR #398, section "What": ISO4 is the 4-bit sibling of ISO3 -- 4.25 bits per value, 68
bytes per 128-value block -- made by the same steps as ISO3 (per 128 values: L2-normalise, rotate
every 4-value group by one fixed unit quaternion, replace each value by the nearest Lloyd-Max
centroid, store the corrected norm ||x|| / ||c||).

Readings where the pages are silent (parity with the original implementation is unpinned):
  * the sixteen centroids are those of the optimal 16-level Lloyd-Max quantiser of a standard
    normal variable, given to 4 decimals as the page gives ISO3's eight, and scaled by 1/sqrt(128);
    the pins check them against that quantiser's fixed point computed from its definition;
  * 68 bytes = 64 bytes of 4-bit codes + a 4-byte norm: the corrected norm is kept in binary32
    (no fp16 rounding), its bytes in two consecutive 16-bit slots of the scales slab (low half
    first);
  * everything else as the ISO3 oracle: one quaternion for every group, the Hamilton product
    q * u, binary32 arithmetic with ``tree_sum`` norms, nearest centroid on binary32 distances with
    the lowest index winning a tie (r = 0 picks index 7), a zero block stores norm 0;
  * codes are a little-endian 4-bit stream: code i in bits [4i, 4i+4), so byte j holds codes 2j
    (low nibble) and 2j + 1 (high nibble).
"""
from __future__ import annotations

import math

import numpy as np

from .iso3 import conjugate, quat_left_mul
from .numerics import F32, tree_sum

BLOCK = 128
CODE_BYTES_PER_BLOCK = 64
LLOYD_MAX_4BIT = (-2.7326, -2.0690, -1.6180, -1.2562, -0.9423, -0.6568, -0.3880, -0.1284,
                  0.1284, 0.3880, 0.6568, 0.9423, 1.2562, 1.6180, 2.0690, 2.7326)


def code_bytes(head_dim: int) -> int:
    return head_dim // BLOCK * CODE_BYTES_PER_BLOCK


def n_scales(head_dim: int) -> int:
    return 2 * (head_dim // BLOCK)          # one binary32 norm per block, in two 16-bit slots


def centroids() -> np.ndarray:
    """Cs[k] = C[k] / sqrt(128), computed in fp64, rounded once to binary32."""
    return np.array([c / math.sqrt(BLOCK) for c in LLOYD_MAX_4BIT], dtype=np.float64).astype(np.float32)


def nearest_centroid(r: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid for each binary32 value (distances in binary32, first minimum wins)."""
    dist = np.abs(np.asarray(r, dtype=np.float32)[..., None] - centroids())
    return np.argmin(dist, axis=-1).astype(np.uint8)


def pack4(codes: np.ndarray) -> np.ndarray:
    """[..., 2k] codes 0..15 -> [..., k] bytes: code 2j in the low nibble of byte j, 2j + 1 in the high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1]).astype(np.uint8)


def norms_to_slots(norms: np.ndarray) -> np.ndarray:
    """binary32 norms [..., nb] -> the scales slab's float16 slots [..., 2 nb] holding their bytes."""
    n = np.ascontiguousarray(np.asarray(norms, dtype="<f4"))
    return n.view(np.uint16).reshape(*n.shape[:-1], 2 * n.shape[-1]).view(np.float16)


def slots_to_norms(slots: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(np.asarray(slots, dtype=np.float16)).view(np.uint16)
    return s.reshape(*s.shape[:-1], s.shape[-1] // 2, 2).copy().view("<f4")[..., 0].astype(np.float32)


def encode_codes(x: np.ndarray, quat):
    """x float32 [..., D] -> (codes uint8 [..., D] in 0..15, norms float32 [..., D/128])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % BLOCK:
        raise ValueError("head_dim must be a multiple of 128")
    blk = x.reshape(*x.shape[:-1], D // BLOCK, BLOCK)
    n = np.sqrt(tree_sum(blk * blk))                                      # ||x||
    safe_n = np.where(n > 0, n, F32(1))[..., None]
    u = np.where((n > 0)[..., None], blk / safe_n, F32(0))                # x / ||x||
    r = quat_left_mul(quat, u.reshape(*u.shape[:-1], BLOCK // 4, 4)).reshape(u.shape)
    codes = nearest_centroid(r)
    cs = centroids()[codes]
    cn = np.sqrt(tree_sum(cs * cs))                                       # ||c||
    norms = (n / cn).astype(np.float32)
    return codes.reshape(x.shape), norms


def encode(x: np.ndarray, quat):
    """x float32 [..., D] -> (packed codes uint8 [..., D/128*64], norm slots float16 [..., 2 D/128])."""
    codes, norms = encode_codes(x, quat)
    return pack4(codes), norms_to_slots(norms)


def decode(packed: np.ndarray, slots: np.ndarray, quat) -> np.ndarray:
    """(packed, norm slots) -> float32 [..., D]: conj(q) * centroid groups, then times the norm."""
    packed = np.asarray(packed)
    nb = packed.shape[-1] // CODE_BYTES_PER_BLOCK
    codes = unpack4(packed).reshape(*packed.shape[:-1], nb, BLOCK)
    c = centroids()[codes]
    w = quat_left_mul(conjugate(quat), c.reshape(*c.shape[:-1], BLOCK // 4, 4)).reshape(c.shape)
    out = w * slots_to_norms(slots)[..., None]
    return out.reshape(*packed.shape[:-1], nb * BLOCK)
