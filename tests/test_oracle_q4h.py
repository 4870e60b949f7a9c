"""Pins for the Hadamard-rotated q4_0 oracle (strata PR #120 "What"/"How"/"Measured";
strata PR #2698 "Not in this PR")."""
import numpy as np
import scipy.linalg

from oracle import q4h, int8_g64
from oracle.numerics import to_f16
from test_oracle_int8 import golden


def test_fwht_matches_library_hadamard():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)).astype(np.float32)
    H = scipy.linalg.hadamard(256).astype(np.float64) / 16.0        # Sylvester order
    ref = v.astype(np.float64) @ H.T
    got = q4h.fwht256(v).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 2e-6 * np.max(np.abs(ref))
    assert np.allclose(q4h.hadamard_f64(v.astype(np.float64)), ref, rtol=0, atol=1e-12)


def test_hadamard_is_orthonormal_and_involutive():
    I = np.eye(256)
    H = q4h.hadamard_f64(I)
    assert np.array_equal(H, H.T)
    assert np.allclose(H @ H, I, atol=1e-15)
    rng = np.random.default_rng(3)
    v = rng.standard_normal((10, 256)).astype(np.float32)
    back = q4h.fwht256(q4h.fwht256(v))
    assert np.max(np.abs(back - v)) < 1e-5
    assert np.allclose(np.linalg.norm(q4h.fwht256(v), axis=1), np.linalg.norm(v, axis=1), rtol=1e-5)


def test_q4_0_worked_example():
    z = np.zeros(32, np.float32)
    # signed max-abs is the first -3.0 (the later +3.0 ties in magnitude), so d = -3/-8 = 0.375
    z[:7] = [-3.0, 1.0, 2.0, 3.0, 0.1875, 0.5625, -0.1875]
    packed, d = q4h.q4_0_encode(z)
    assert d.view(np.uint16)[0] == 0x3600           # fp16 0.375
    codes = q4h.unpack_nibbles(packed)
    # -3/.375=-8 -> 0; 1/.375=2.67 -> 3 -> 11; 2/.375=5.33 -> 5 -> 13; 3/.375=8 -> 16 -> clamp 15;
    # .1875/.375=0.5 -> tie to even 0 -> 8; .5625/.375=1.5 -> 2 -> 10; -0.5 -> -0 -> 8
    assert list(codes[:7]) == [0, 11, 13, 15, 8, 10, 8]
    assert np.all(codes[7:] == 8)
    assert packed[0] == 0xB0 and packed[1] == 0xFD     # low nibble = even element
    z2 = -z
    _, d2 = q4h.q4_0_encode(z2)
    assert d2[0] == np.float16(-0.375)


def test_q4_0_zero_block():
    packed, d = q4h.q4_0_encode(np.zeros(64, np.float32))
    assert np.all(packed == 0x88) and np.all(d == 0) and not np.any(np.signbit(d))


def test_q4_0_brute_force_and_bound():
    rng = np.random.default_rng(4)
    z = (rng.standard_normal((400, 256)) * rng.uniform(0.01, 20, (400, 1))).astype(np.float32)
    packed, d = q4h.q4_0_encode(z)
    codes = q4h.unpack_nibbles(packed).reshape(400, 8, 32).astype(np.int64)
    blk = z.reshape(400, 8, 32).astype(np.float64)
    first = np.argmax(np.abs(blk), axis=-1)
    m = np.take_along_axis(blk, first[..., None], -1)[..., 0]
    d32 = m / -8.0
    cand = np.arange(16)
    err = np.abs(blk[..., None] - (cand - 8) * d32[..., None, None])
    best = cand[np.argmin(err, axis=-1)]
    frac = np.abs(blk / d32[..., None]) % 1.0
    clear = np.abs(frac - 0.5) > 1e-4
    assert np.array_equal(codes[clear], best[clear])
    y = q4h.q4_0_decode(packed, d).reshape(400, 8, 32).astype(np.float64)
    df = d.astype(np.float64)
    clamped = blk / d32[..., None] > 7.5
    bound = np.abs(d32)[..., None] / 2 + 8 * np.abs(d32 - df)[..., None] + 1e-6 * np.abs(m)[..., None]
    assert np.all(np.abs(y - blk)[~clamped] <= np.broadcast_to(bound, blk.shape)[~clamped])
    assert np.all(np.abs(y - blk)[clamped] <= (np.abs(m)[..., None] / 8 + 8 * np.abs(d32 - df)[..., None]
                                              + 1e-6 * np.abs(m)[..., None]).repeat(32, -1)[clamped])
    # the signed max element reconstructs to m up to the fp16 rounding of d
    top = np.take_along_axis(y, first[..., None], -1)[..., 0]
    assert np.allclose(top, -8 * df)


def test_bytes_match_the_pages():
    gv = golden()
    D, hkv = 256, 2
    v_head = q4h.code_bytes(D) + 2 * q4h.n_scales(D)
    k_head = int8_g64.code_bytes(D) + 2 * int8_g64.n_scales(D)
    assert v_head == gv["q4_0_v_gather_bytes_per_head_cell"]
    assert hkv * (k_head + v_head) == gv["k8v4_bytes_per_cell_kv"]
    assert hkv * 2 * v_head == gv["q4_0_bytes_per_cell_kv"]
    assert hkv * 2 * k_head == gv["int8_bytes_per_cell_kv"]
    # the measured cache sizes at 131k keep the same ratio to two decimals
    assert abs(gv["k8v4_kv_gb_at_131k"] / gv["int8_kv_gb_at_131k"] - 816 / 1056) < 0.005


def test_encode_rotates_first():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((3, 2, 256)).astype(np.float32)
    p1, d1 = q4h.encode(v)
    p2, d2 = q4h.q4_0_encode(q4h.fwht256(v))
    assert np.array_equal(p1, p2) and np.array_equal(d1.view(np.uint16), d2.view(np.uint16))
    # back in the original basis the error stays at q4_0 level (orthonormal rotation preserves it)
    back = q4h.decode(p1, d1)
    rel = np.linalg.norm(back - v, axis=-1) / np.linalg.norm(v, axis=-1)
    assert np.all(rel < 0.2)
    assert to_f16(np.float32(0.375)) == np.float16(0.375)
