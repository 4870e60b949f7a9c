"""Pins for the unquantised FP32 store of the oracle and for attention over the single-store modes
(strata PR #2698: FP32 caches of 2 KiB per cell per store at head_dim 256; `k8v32` / `k32v8` quantise
one store only)."""
import math

import numpy as np

from oracle import attention, f32, int8_g64, paged
from oracle.numerics import bf16_to_f32
from test_oracle_int8 import golden


def test_bytes_per_cell_match_the_pages():
    gv = golden()
    D, hkv = 256, 2
    fp32 = (f32.code_bytes(D) + 2 * f32.n_scales(D)) * hkv
    int8 = (int8_g64.code_bytes(D) + 2 * int8_g64.n_scales(D)) * hkv
    assert fp32 == gv["fp32_bytes_per_cell_one_store_d256_hkv2"]
    # one store quantised: between both stores int8 and both FP32
    assert 2 * int8 < int8 + fp32 < 2 * fp32


def test_cells_are_little_endian_binary32():
    # IEEE 754 binary32 patterns: 1.0 = 0x3f800000, -2.5 = 0xc0200000, -0.0 = 0x80000000, and the
    # smallest positive bf16 subnormal 2^-133 = 0x00010000
    x = np.array([1.0, -2.5, -0.0, 2.0 ** -133], np.float32)
    codes, scales = f32.encode(x)
    assert scales.shape == (0,)
    assert codes.tolist() == [0x00, 0x00, 0x80, 0x3f, 0x00, 0x00, 0x20, 0xc0, 0x00, 0x00, 0x00, 0x80,
                              0x00, 0x00, 0x01, 0x00]


def test_bf16_values_round_trip_exactly():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7f80) != 0x7f80]                 # every finite bf16, both signs
    x = bf16_to_f32(finite).reshape(-1, 128)[:, None, :]
    codes, scales = paged.encode_cells("f32", x)
    back = paged.decode_cells("f32", codes, scales)
    assert np.array_equal(back.view(np.uint32), x.view(np.uint32))


def _brute_attention(q, K, V, sm_scale):
    """Softmax attention of one query row, written out with Python loops."""
    s = [sm_scale * sum(float(q[d]) * float(K[j][d]) for d in range(len(q))) for j in range(len(K))]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    den = sum(w)
    return [sum(w[j] * float(V[j][d]) for j in range(len(K))) / den for d in range(len(q))]


def _paged_pair(fmt_k, fmt_v, k_bits, v_bits, perm):
    """One sequence of L tokens on pages `perm`: oracle stores of both formats."""
    L, hkv, D = k_bits.shape
    n_pages = len(perm)
    bt = np.asarray(perm, np.int32)[None, :]
    sk = paged.Store.empty(fmt_k, n_pages, hkv, 16, D)
    sv = paged.Store.empty(fmt_v, n_pages, hkv, 16, D)
    pos = np.arange(L)
    paged.append(sk, bt, np.zeros(L, int), pos, k_bits, 16)
    paged.append(sv, bt, np.zeros(L, int), pos, v_bits, 16)
    return sk, sv, bt


def test_single_store_modes_reduce_to_plain_attention():
    """k8v32, k32v8 and FP32 K + V through a shuffled page table against softmax attention written out
    over the stored values (FP32: the bf16 inputs; int8: code x scale)."""
    rng = np.random.default_rng(5)
    L, hkv, D, hq = 37, 2, 128, 4
    k = rng.standard_normal((L, hkv, D)).astype(np.float32)
    v = rng.standard_normal((L, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, hq, D)).astype(np.float32)
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    k_bits, v_bits, q_bits = to_bits(k), to_bits(v), to_bits(q)
    kf, vf, qf = bf16_to_f32(k_bits), bf16_to_f32(v_bits), bf16_to_f32(q_bits)
    k8 = int8_g64.decode(*int8_g64.encode(kf)).astype(np.float32)
    v8 = int8_g64.decode(*int8_g64.encode(vf)).astype(np.float32)
    perm = [2, 0, 3, 1]
    scale = 1.0 / math.sqrt(D)
    for fk, fv, K, V in (("int8", "f32", k8, vf), ("f32", "int8", kf, v8), ("f32", "f32", kf, vf)):
        sk, sv, bt = _paged_pair(fk, fv, k_bits, v_bits, perm)
        got = attention.decode(sk, sv, bt, np.array([L]), q_bits, 16, scale)
        for h in range(hq):
            kh = h // (hq // hkv)
            ref = _brute_attention(qf[0, 0, h], K[:, kh], V[:, kh], scale)
            assert np.allclose(got[0, 0, h], ref, rtol=1e-6, atol=1e-6), (fk, fv, h)
