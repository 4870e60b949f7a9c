"""Pins for the INT8 group-64 oracle (strata PR #2698 "What it does"; strata PR #120 "Tests")."""
import os

import numpy as np

from oracle import int8_g64
from oracle.numerics import to_f16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_byte_counts.txt")


def golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()[:2]
        vals[k] = float(v)
    return vals


def test_ties_to_even_worked_example():
    # A group whose max-abs is 127 has scale exactly 1.0, so x/scale = x and the printed
    # ties-to-even rule decides: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0, 1.5 -> 2, -0.5 -> -0.
    g = np.zeros(64, np.float32)
    g[:7] = [2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 127.0]
    codes, scales = int8_g64.encode(g)
    assert list(codes[:7]) == [2, 4, -2, 0, 2, 0, 127]
    assert scales.view(np.uint16)[0] == 0x3C00   # fp16 1.0


def test_scale_is_absmax_over_127_stored_fp16():
    g = np.zeros(64, np.float32)
    g[5] = -1.0
    codes, scales = int8_g64.encode(g)
    assert scales.view(np.uint16)[0] == 0x2008   # fp16(1/127), rounded to nearest even
    assert codes[5] == -127 and np.count_nonzero(codes) == 1


def test_zero_group_and_independent_groups():
    x = np.zeros(128, np.float32)
    x[64:] = np.linspace(-2, 2, 64, dtype=np.float32)
    codes, scales = int8_g64.encode(x)
    assert scales[0] == 0 and not np.signbit(scales[0]) and np.all(codes[:64] == 0)
    assert scales[1] == to_f16(np.float32(2.0) / np.float32(127))
    assert codes[64] == -127 and codes[127] == 127


def test_codes_are_brute_force_nearest_and_bounds_hold():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((500, 256)) * rng.uniform(0.01, 50, (500, 1))).astype(np.float32)
    codes, scales = int8_g64.encode(x)
    g = x.reshape(500, 4, 64).astype(np.float64)
    s32 = (np.abs(x.reshape(500, 4, 64)).max(-1) / np.float32(127)).astype(np.float64)
    cand = np.arange(-127, 128)
    err = np.abs(g[..., None] - cand * s32[..., None, None])          # fp64 brute force over all codes
    best = cand[np.argmin(err, axis=-1)]
    frac = np.abs(g / s32[..., None]) % 1.0
    clear = np.abs(frac - 0.5) > 1e-4                                 # away from rounding ties
    assert np.array_equal(codes.reshape(500, 4, 64)[clear], best[clear])
    # max-abs element of every group maps to +-127
    am = np.argmax(np.abs(g), axis=-1)
    top = np.take_along_axis(codes.reshape(500, 4, 64), am[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    # round-trip: |x - code*fp16(s)| <= s/2 + 127*|s - fp16(s)|  (+ one ulp of slack)
    xh = int8_g64.decode(codes, scales).reshape(500, 4, 64).astype(np.float64)
    sf = scales.astype(np.float64)
    bound = s32 / 2 + 127 * np.abs(s32 - sf) + 1e-6 * s32
    assert np.all(np.abs(xh - g) <= bound[..., None])
    assert np.all(bound <= 0.5621 * s32 + 1e-6 * s32)


def test_bytes_per_cell_match_the_pages():
    gv = golden()
    D, hkv = 256, 2
    per_head = int8_g64.code_bytes(D) + 2 * int8_g64.n_scales(D)
    assert per_head * hkv == gv["int8_bytes_per_cell_one_store_d256_hkv2"]
    assert 4 * D * hkv == gv["fp32_bytes_per_cell_one_store_d256_hkv2"]
    assert round(gv["fp32_bytes_per_cell_one_store_d256_hkv2"] / (per_head * hkv), 1) == gv["int8_vs_fp32_ratio_approx"]
    assert 2 * per_head * hkv == gv["int8_bytes_per_cell_kv"]
