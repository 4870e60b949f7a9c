"""GPU parity of decode / verify attention over Hadamard-rotated q4_0 K and V stores, through the C ABI.

The kernel rotates the query by H and contracts it with the stored (rotated) K codes, accumulates V in
the rotated basis and rotates each split's partial back; the oracle dequantises every cell, rotates K
and V back in fp64 and runs fp64 attention.  Every case checks the slabs byte for byte against the
oracle's encoding and the attention to max-abs 1e-3 with cosine > 0.9999 over the tensor and every row.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, assert_slabs_equal, dev_bf16, dev_i32, gpu_append, gpu_cache,
                          oracle_decode, oracle_stores)

pytestmark = pytest.mark.gpu


def run_decode(w, head_map=None):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn(cache, pages, dev_bf16(w.q), q_lens=q_lens, head_map=head_map, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return cache, out.cpu().numpy()


def check(w, head_map=None):
    print(f"[q4 decode] {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} n_q={w.n_q} "
          f"lens={list(w.seq_lens)[:8]}", flush=True)
    cache, got = run_decode(w, head_map)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(got, oracle_decode(w, sk, sv, head_map=head_map))
    print(f"[q4 decode] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)
    return m


def q4(lens, seed, **kw):
    return synth.ragged_decode("q4h", "q4h", lens, seed=seed, head_dim=256, **kw)


def test_q4_decode_ragged_lengths():
    """Lengths on and around page edges and a few splits deep; 4 query rows per KV head."""
    check(q4([1, 15, 16, 17, 300, 1024, 2100], 81, n_q_heads=8, n_kv_heads=2))


def test_q4_decode_64_page_splits():
    """Four sequences over eight KV heads: 9 x 8 x 4 = 288 splits of 64 pages fill more than one
    workgroup per CU, so the plan keeps 64-page splits (the other launch shape)."""
    check(q4([9000, 8200, 4100, 9000], 82, n_q_heads=16, n_kv_heads=8))


def test_q4_decode_eight_rows():
    check(q4([5, 700, 4100], 82, n_q_heads=16, n_kv_heads=2))


@pytest.mark.parametrize("n_q,hq", [(2, 8), (3, 8), (2, 16)])
def test_q4_verify_window(n_q, hq):
    """Verify windows with per-query causal lengths: 8 rows (hi / lo in one MFMA's columns), 12 and
    16 rows (separate hi and lo MFMAs)."""
    back = list(range(n_q - 1, -1, -1))
    check(q4([40, 17, 1000, 2049], 83 + n_q + hq, n_q=n_q, q_len_back=back, n_q_heads=hq, n_kv_heads=2))


def test_q4_verify_window_eight_wave_shapes():
    """16 rows (separate hi / lo MFMAs) over 8 KV heads in the 8-wave launch shapes: 20,000 tokens give
    20 splits of 64 pages per KV head (160 workgroups, more than half of the CUs: 64-page splits),
    9,000 tokens 9 (72: 32-page splits)."""
    for L, seed in ((20000, 86), (9000, 87)):
        check(q4([L], seed, n_q=2, q_len_back=[1, 0], n_q_heads=64, n_kv_heads=8))


def test_q4_decode_head_map_and_idle_kv_heads():
    """Uneven groups through an explicit map; KV heads 1 and 3 (the last) serve no query head."""
    check(q4([33, 500], 84, n_q_heads=6, n_kv_heads=4), head_map=[2, 0, 2, 0, 2, 2])


@pytest.mark.parametrize("lens", [[0, 5, 300], [0, 2000, 17]])
def test_q4_decode_empty_sequence(lens):
    """A sequence with no cells gets zeros, from its only split (one split: no combine launch) or
    from the combine."""
    check(q4(lens, 90 + lens[1], n_q_heads=8, n_kv_heads=2))


def test_q4_decode_mha_and_mqa():
    check(q4([90, 260], 85, n_q_heads=4, n_kv_heads=4))
    check(q4([90, 260], 86, n_q_heads=8, n_kv_heads=1))


def test_q4_decode_outlier_keys():
    """K with outlier channels (the rotation spreads them over all 256 values of the cell)."""
    check(synth.moe_q4h_decode(ctx=3000, seed=87))


def test_q4_decode_rising_scores_move_the_reference_max():
    from oracle.numerics import bf16_to_f32
    L = 3000
    w = q4([L], 88, n_q_heads=8, n_kv_heads=2)
    k = bf16_to_f32(w.k[0]).copy()
    q = bf16_to_f32(w.q)
    qdir = q[0, :, :4].mean(axis=(0, 1))
    qdir /= np.linalg.norm(qdir)
    ramp = np.linspace(0.0, 120.0, L, dtype=np.float32)
    ramp[1500:] += 80.0
    k[:, 0, :] += ramp[:, None] * qdir[None, :]
    w.k[0] = synth.bf16_bits(k)
    check(w)


def test_q4_decode_deterministic():
    w = synth.moe_q4h_decode(ctx=5000, seed=89)
    _, a = run_decode(w)
    _, b = run_decode(w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_q4_decode_moe_full_size_131072():
    """The q4_0 benchmark's workload at full size, in the launch configuration the benchmark times."""
    check(synth.moe_q4h_decode(ctx=131072))
