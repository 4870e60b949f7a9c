"""ISO3 (IsoQuant 3-bit) cache cells (oracle; test infrastructure only).

Method (FreeToken PR #398, section "What"): per block of 128 values of a head
vector -- L2-normalise, rotate every 4-value group by one fixed unit quaternion,
replace each value by the nearest 3-bit Lloyd-Max centroid, and store the
corrected norm ||x|| / ||c|| (c = the vector of chosen centroids), so that the
dequantised block keeps the input's norm.  3.125 bits per value: 48 bytes of
codes plus a 2-byte FP16 norm per 128 values (same page, section "What").

The eight centroids are those of the optimal 3-bit Lloyd-Max quantiser for a
standard normal variable, {+-0.2451, +-0.7560, +-1.3440, +-2.1520}, scaled by
1/sqrt(128) because a normalised 128-vector has per-value variance 1/128.

Readings where the pages are silent:
  * one quaternion q = (w, x, y, z) for every group, block, head, token, K and V;
    the group (u0, u1, u2, u3) is the quaternion (w, x, y, z) and the rotation is
    the Hamilton product q * u (left multiplication); dequantisation applies the
    conjugate (w, -x, -y, -z) the same way;
  * binary32 throughout: the squared norm is a ``tree_sum`` of x_i*x_i, then sqrt;
    u = x / n; each Hamilton-product component is evaluated left to right as
    written in ``quat_left_mul``;
  * "nearest" is decided on binary32 distances |r - Cs[k]|, the lowest index
    winning a tie (so r = 0 picks index 3, the centroid -0.2451/sqrt(128));
  * Cs[k] = fp32(C[k] / sqrt(128)) computed in fp64 and rounded once;
  * the stored norm is fp16(n / ||Cs[codes]||) with ||.|| a ``tree_sum`` of squares
    then sqrt; a zero block stores norm 0 (and codes 3);
  * dequantisation rotates the centroids by the conjugate first, then multiplies
    by the stored norm;
  * codes are a little-endian bit stream, code i in bits [3i, 3i+3): eight codes
    per three bytes; norms live in their own FP16 slab.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import F32, to_f16, tree_sum

BLOCK = 128
CODE_BYTES_PER_BLOCK = 48
LLOYD_MAX_3BIT = (-2.1520, -1.3440, -0.7560, -0.2451, 0.2451, 0.7560, 1.3440, 2.1520)


def code_bytes(head_dim: int) -> int:
    return head_dim // BLOCK * CODE_BYTES_PER_BLOCK


def n_scales(head_dim: int) -> int:
    return head_dim // BLOCK


def centroids() -> np.ndarray:
    """Cs[k] = C[k] / sqrt(128), computed in fp64, rounded once to binary32."""
    return np.array([c / math.sqrt(BLOCK) for c in LLOYD_MAX_3BIT], dtype=np.float64).astype(np.float32)


def conjugate(quat) -> np.ndarray:
    w, x, y, z = np.asarray(quat, dtype=np.float32)
    return np.array([w, -x, -y, -z], dtype=np.float32)


def quat_left_mul(quat, g: np.ndarray) -> np.ndarray:
    """Hamilton product quat * g for every 4-vector g[..., 0:4] = (w, x, y, z), binary32, left to right."""
    w, x, y, z = (F32(v) for v in np.asarray(quat, dtype=np.float32))
    a, b, c, d = (np.asarray(g[..., i], dtype=np.float32) for i in range(4))
    r0 = ((w * a - x * b) - y * c) - z * d
    r1 = ((w * b + x * a) + y * d) - z * c
    r2 = ((w * c - x * d) + y * a) + z * b
    r3 = ((w * d + x * c) - y * b) + z * a
    return np.stack([r0, r1, r2, r3], axis=-1)


def nearest_centroid(r: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid for each binary32 value (distances in binary32, first minimum wins)."""
    cs = centroids()
    dist = np.abs(np.asarray(r, dtype=np.float32)[..., None] - cs)
    return np.argmin(dist, axis=-1).astype(np.uint8)


def pack3(codes: np.ndarray) -> np.ndarray:
    """[..., 128] codes 0..7 -> [..., 48] bytes; code i occupies bits 3i..3i+2 of a little-endian stream."""
    c = np.asarray(codes, dtype=np.uint32)
    c = c.reshape(*c.shape[:-1], c.shape[-1] // 8, 8)
    word = np.zeros(c.shape[:-1], dtype=np.uint32)
    for m in range(8):
        word |= c[..., m] << np.uint32(3 * m)
    out = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
    return out.reshape(*c.shape[:-2], c.shape[-2] * 3).astype(np.uint8)


def unpack3(packed: np.ndarray) -> np.ndarray:
    """[..., 48k] bytes -> [..., 128k] codes 0..7."""
    p = np.asarray(packed, dtype=np.uint32)
    p = p.reshape(*p.shape[:-1], p.shape[-1] // 3, 3)
    word = p[..., 0] | (p[..., 1] << np.uint32(8)) | (p[..., 2] << np.uint32(16))
    codes = np.stack([(word >> np.uint32(3 * m)) & np.uint32(7) for m in range(8)], axis=-1)
    return codes.reshape(*codes.shape[:-2], codes.shape[-2] * 8).astype(np.uint8)


def encode_codes(x: np.ndarray, quat):
    """x float32 [..., D] -> (codes uint8 [..., D] in 0..7, norms float16 [..., D/128])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % BLOCK:
        raise ValueError("head_dim must be a multiple of 128")
    blk = x.reshape(*x.shape[:-1], D // BLOCK, BLOCK)
    n = np.sqrt(tree_sum(blk * blk))                                      # ||x||
    safe_n = np.where(n > 0, n, F32(1))[..., None]
    u = np.where((n > 0)[..., None], blk / safe_n, F32(0))                # x / ||x||
    r = quat_left_mul(quat, u.reshape(*u.shape[:-1], BLOCK // 4, 4))      # rotate each 4-group
    r = r.reshape(u.shape)
    codes = nearest_centroid(r)
    cs = centroids()[codes]
    cn = np.sqrt(tree_sum(cs * cs))                                       # ||c||
    norms = to_f16(n / cn)
    return codes.reshape(x.shape), norms


def encode(x: np.ndarray, quat):
    """x float32 [..., D] -> (packed codes uint8 [..., D/128*48], norms float16 [..., D/128])."""
    codes, norms = encode_codes(x, quat)
    D = codes.shape[-1]
    packed = pack3(codes.reshape(*codes.shape[:-1], D // BLOCK, BLOCK))
    return packed.reshape(*codes.shape[:-1], D // BLOCK * CODE_BYTES_PER_BLOCK), norms


def decode(packed: np.ndarray, norms: np.ndarray, quat) -> np.ndarray:
    """(packed, norms) -> float32 [..., D]: conj(q) * centroid groups, then times the stored norm."""
    packed = np.asarray(packed)
    nb = packed.shape[-1] // CODE_BYTES_PER_BLOCK
    codes = unpack3(packed.reshape(*packed.shape[:-1], nb, CODE_BYTES_PER_BLOCK))   # [..., nb, 128]
    c = centroids()[codes]
    w = quat_left_mul(conjugate(quat), c.reshape(*c.shape[:-1], BLOCK // 4, 4)).reshape(c.shape)
    out = w * np.asarray(norms).astype(np.float32)[..., None]
    return out.reshape(*packed.shape[:-1], nb * BLOCK)
