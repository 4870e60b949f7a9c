"""Pins for the ISO4 oracle (FreeToken PR #398, section "What": ISO4 at 4.25 bits per value, 68 bytes per
128-value block, made like ISO3).  The page does not list ISO4's sixteen centroids; the oracle takes the
16-level Lloyd-Max quantiser of a standard normal variable, and these pins check it against that
quantiser computed here from its definition (centroid and midpoint conditions)."""
import math

import numpy as np
from scipy.stats import norm

from oracle import iso3, iso4, paged
from synth import random_quaternion
from test_oracle_int8 import golden


def lloyd_max_normal(levels: int) -> np.ndarray:
    """Fixed point of the Lloyd iteration for N(0, 1): thresholds at midpoints, levels at the
    conditional means of their cells."""
    c = norm.ppf((np.arange(levels) + 0.5) / levels)
    for _ in range(10000):
        t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        new = (norm.pdf(t[:-1]) - norm.pdf(t[1:])) / (norm.cdf(t[1:]) - norm.cdf(t[:-1]))
        if np.max(np.abs(new - c)) < 1e-14:
            return new
        c = new
    return c


def test_levels_are_the_16_level_lloyd_max_quantiser():
    exact = lloyd_max_normal(16)
    assert np.max(np.abs(np.array(iso4.LLOYD_MAX_4BIT) - exact)) <= 5e-5      # 4 decimals
    # the page's ISO3 list comes from the 8-level quantiser (its last digits deviate by up to 1e-4)
    assert np.max(np.abs(np.array(iso3.LLOYD_MAX_3BIT) - lloyd_max_normal(8))) <= 1.2e-4
    cs = iso4.centroids()
    assert np.all(np.diff(cs) > 0) and np.array_equal(cs[:8], -cs[:7:-1])


def test_bytes_per_block_match_the_page():
    gv = golden()
    D = 128
    per_block = iso4.code_bytes(D) + 2 * iso4.n_scales(D)
    assert per_block == gv["iso4_bytes_per_128_block"]
    assert per_block * 8 / 128 == gv["iso4_bits_per_value"]
    assert round(2 * 128 / per_block, 1) == gv["iso4_vs_bf16_ratio_approx"]
    assert paged.cell_bytes("iso4", 256) == (128, 4)


def test_nibble_stream_and_norm_slots():
    assert iso4.pack4(np.array([1, 2, 15, 0], np.uint8)).tolist() == [0x21, 0x0F]
    c = np.random.default_rng(3).integers(0, 16, size=(5, 128)).astype(np.uint8)
    assert np.array_equal(iso4.unpack4(iso4.pack4(c)), c)
    # binary32 1.0 = 0x3f800000: low half first
    assert iso4.norms_to_slots(np.array([1.0], np.float32)).view(np.uint16).tolist() == [0x0000, 0x3F80]
    n = np.random.default_rng(4).random((3, 2)).astype(np.float32)
    assert np.array_equal(iso4.slots_to_norms(iso4.norms_to_slots(n)), n)


def test_codes_are_brute_force_nearest_and_zero_block():
    rng = np.random.default_rng(8)
    q = random_quaternion(9)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    codes, norms = iso4.encode_codes(x, q)
    cs = iso4.centroids()
    for i in range(3):
        n = math.sqrt(float(np.sum(x[i].astype(np.float64) ** 2)))
        u = (x[i] / np.float32(n)).reshape(32, 4)
        r = iso3.quat_left_mul(q, u).reshape(128)
        for d in range(128):
            dist = [abs(float(np.float32(r[d]) - cs[k])) for k in range(16)]
            assert codes[i, d] == int(np.argmin(dist))
    z_codes, z_norms = iso4.encode_codes(np.zeros((1, 128), np.float32), q)
    assert np.all(z_codes == 7) and z_norms[0, 0] == 0.0


def test_dequantisation_keeps_the_norm_and_the_quantiser_distortion():
    """Norm-preserving dequantisation ("What": the corrected norm), and a per-value error that matches
    the 16-level quantiser's distortion for Gaussian inputs (a wrong rotation, level or code order
    would not)."""
    rng = np.random.default_rng(10)
    q = random_quaternion(11)
    x = rng.standard_normal((400, 256)).astype(np.float32)
    packed, slots = iso4.encode(x, q)
    y = iso4.decode(packed, slots, q)
    xb = x.reshape(400, 2, 128).astype(np.float64)
    yb = y.reshape(400, 2, 128).astype(np.float64)
    assert np.allclose(np.linalg.norm(yb, axis=-1), np.linalg.norm(xb, axis=-1), rtol=2e-6)
    # distortion of the unit-variance quantiser: E[(X - Q(X))^2] for X ~ N(0, 1)
    ex = lloyd_max_normal(16)
    t = np.concatenate([[-np.inf], (ex[:-1] + ex[1:]) / 2, [np.inf]])
    p = norm.cdf(t[1:]) - norm.cdf(t[:-1])
    d = 1.0 - float(np.sum(p * ex * ex))
    # the rotation is orthogonal, so the error per value of the normalised block is that of the
    # quantiser on (nearly Gaussian) values of variance 1/128, up to the norm correction
    err = np.mean(((yb - xb) / np.linalg.norm(xb, axis=-1, keepdims=True)) ** 2) * 128
    assert 0.85 * d < err < 1.15 * d, (err, d)
