"""Pins for the ISO3 oracle (FreeToken PR #398, sections "What" and "Why")."""
import math

import numpy as np

from oracle import iso3
from synth import random_quaternion
from test_oracle_int8 import golden

ONE = np.array([1, 0, 0, 0], np.float32)
I_ = np.array([0, 1, 0, 0], np.float32)
J_ = np.array([0, 0, 1, 0], np.float32)
K_ = np.array([0, 0, 0, 1], np.float32)


def qm(a, b):
    return iso3.quat_left_mul(a, np.asarray(b, np.float32)[None, :])[0]


def test_hamilton_rules():
    # i^2 = j^2 = k^2 = ijk = -1, ij = k, jk = i, ki = j, ji = -k
    for u in (I_, J_, K_):
        assert np.array_equal(qm(u, u), -ONE)
    assert np.array_equal(qm(I_, J_), K_)
    assert np.array_equal(qm(J_, K_), I_)
    assert np.array_equal(qm(K_, I_), J_)
    assert np.array_equal(qm(J_, I_), -K_)
    assert np.array_equal(qm(qm(I_, J_), K_), -ONE)
    assert np.array_equal(qm(ONE, I_), I_)


def test_left_multiplication_is_bilinear_and_norm_preserving():
    rng = np.random.default_rng(6)
    q = random_quaternion(7)
    v = rng.standard_normal((100, 4)).astype(np.float32)
    basis = [ONE, I_, J_, K_]
    # expand q*v over the basis products fixed by Hamilton's rules (fp64)
    ref = np.zeros((100, 4))
    for a in range(4):
        for b in range(4):
            ref += float(q[a]) * v[:, b:b + 1].astype(np.float64) * qm(basis[a], basis[b]).astype(np.float64)
    got = iso3.quat_left_mul(q, v).astype(np.float64)
    assert np.allclose(got, ref, rtol=0, atol=1e-6)
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(v, axis=1), rtol=1e-6)
    back = iso3.quat_left_mul(iso3.conjugate(q), iso3.quat_left_mul(q, v))
    assert np.allclose(back, v, atol=1e-5)


def test_centroids_satisfy_lloyd_max_conditions():
    # For N(0,1): each centroid is the conditional mean of its cell, cell edges at the midpoints.
    C = np.array(iso3.LLOYD_MAX_3BIT)
    assert np.all(np.diff(C) > 0) and np.allclose(C, -C[::-1])
    t = np.concatenate([[-np.inf], (C[1:] + C[:-1]) / 2, [np.inf]])
    phi = lambda x: 0.0 if np.isinf(x) else math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    Phi = lambda x: (0.0 if x < 0 else 1.0) if np.isinf(x) else 0.5 * (1 + math.erf(x / math.sqrt(2)))
    for k in range(8):
        mean = (phi(t[k]) - phi(t[k + 1])) / (Phi(t[k + 1]) - Phi(t[k]))
        assert abs(mean - C[k]) < 1e-4
    cs = iso3.centroids()
    assert cs.dtype == np.float32 and np.allclose(cs * math.sqrt(128), C, rtol=1e-7)


def test_identity_quaternion_is_scalar_nearest_centroid():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    codes, norms = iso3.encode_codes(x, ONE)
    u = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    C = np.array(iso3.LLOYD_MAX_3BIT) / math.sqrt(128)
    best = np.argmin(np.abs(u[..., None] - C), axis=-1)
    mids = (C[1:] + C[:-1]) / 2
    clear = np.min(np.abs(u[..., None] - mids), axis=-1) > 1e-6
    assert np.array_equal(codes[clear], best[clear])


def test_norm_preserving_dequant_and_distortion():
    rng = np.random.default_rng(9)
    q = random_quaternion(10)
    x = rng.standard_normal((2000, 256)).astype(np.float32)
    packed, norms = iso3.encode(x, q)
    xh = iso3.decode(packed, norms, q).astype(np.float64)
    xb = x.reshape(2000, 2, 128).astype(np.float64)
    xhb = xh.reshape(2000, 2, 128)
    nx, nxh = np.linalg.norm(xb, axis=-1), np.linalg.norm(xhb, axis=-1)
    assert np.all(np.abs(nxh / nx - 1) < 2.0 ** -11 + 1e-5)       # only the fp16 norm rounding
    # The 3-bit Lloyd-Max quantiser of N(0,1) has mean-squared error ~0.0345; with the
    # norm correction the per-block relative error lands close to it.
    rel = np.mean(np.sum((xhb - xb) ** 2, -1) / np.sum(xb ** 2, -1))
    assert 0.025 < rel < 0.045


def test_zero_block():
    q = random_quaternion(11)
    x = np.zeros((1, 128), np.float32)
    codes, norms = iso3.encode_codes(x, q)
    assert np.all(codes == 3) and norms[0, 0] == 0
    packed, norms = iso3.encode(x, q)
    assert np.all(iso3.decode(packed, norms, q) == 0)


def test_pack3_worked_example():
    # codes 0..7 as a little-endian 3-bit stream: sum k << 3k = 0xFAC688
    codes = np.zeros(128, np.uint8)
    codes[:8] = np.arange(8)
    p = iso3.pack3(codes)
    assert p.shape == (48,) and list(p[:3]) == [0x88, 0xC6, 0xFA] and np.all(p[3:] == 0)
    rng = np.random.default_rng(12)
    c = rng.integers(0, 8, (5, 3, 128)).astype(np.uint8)
    assert np.array_equal(iso3.unpack3(iso3.pack3(c)), c)


def test_bytes_match_the_pages():
    gv = golden()
    per_block = iso3.CODE_BYTES_PER_BLOCK + 2
    assert per_block == gv["iso3_bytes_per_128_block"]
    assert per_block * 8 / 128 == gv["iso3_bits_per_value"]
    assert round(128 * 2 / per_block, 1) == gv["iso3_vs_bf16_ratio_approx"]
    # 10 full-attention layers, K and V, 2 KV heads x head_dim 256 (= 512 values per store per layer)
    layers, values = 10, 512
    assert layers * 2 * values * 2 == gv["bf16_kv_bytes_per_token_10_layers"]
    assert layers * 2 * (values // 128) * per_block == gv["iso3_kv_bytes_per_token_10_layers"]
    assert iso3.code_bytes(256) == 96 and iso3.n_scales(256) == 2
