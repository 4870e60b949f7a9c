"""GPU parity of decode / verify attention over ISO3 K and V stores, through the C ABI.

The query is rotated by the format's quaternion, the codes enter the MFMAs through a table of
level pairs, values accumulate in the rotated basis and each split's partial is rotated back; the
oracle dequantises every cell (conjugate rotation, times the norm) and runs fp64 attention.  Every
case checks the slabs byte for byte against the oracle's encoding and the attention to max-abs
1e-3 with cosine > 0.9999 over the tensor and every row.
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


def check(w, head_map=None, slabs=True):
    print(f"[iso3 decode] {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} n_q={w.n_q} "
          f"lens={list(w.seq_lens)[:8]}", flush=True)
    cache, got = run_decode(w, head_map)
    sk, sv = oracle_stores(w)
    if slabs:
        assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(got, oracle_decode(w, sk, sv, head_map=head_map))
    print(f"[iso3 decode] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)
    return m


@pytest.mark.parametrize("D", [128, 256])
def test_iso3_decode_ragged_lengths(D):
    """Lengths on and around page edges and a few splits deep; 4 query rows per KV head."""
    check(synth.ragged_decode("iso3", "iso3", [1, 15, 16, 17, 300, 1024, 2100], seed=61 + D, n_q_heads=8,
                              n_kv_heads=2, head_dim=D))


@pytest.mark.parametrize("D", [128, 256])
def test_iso3_decode_64_page_splits(D):
    """Four sequences over eight KV heads: 9 x 8 x 4 = 288 splits of 64 pages fill more than one
    workgroup per CU, so the plan keeps 64-page splits (the other launch shape: 4 waves x 16 pages)."""
    check(synth.ragged_decode("iso3", "iso3", [9000, 8200, 4100, 9000], seed=83, n_q_heads=16, n_kv_heads=8,
                              head_dim=D))


def test_iso3_decode_eight_rows_head_dim_256():
    """8 query rows per KV head: the hi / lo parts fill MFMA columns 0-7 and 8-15."""
    check(synth.ragged_decode("iso3", "iso3", [5, 700, 4100], seed=62, n_q_heads=16, n_kv_heads=2, head_dim=256))


@pytest.mark.parametrize("n_q,hq,D", [(3, 8, 128), (2, 16, 256), (2, 4, 128)])
def test_iso3_verify_windows(n_q, hq, D):
    """Verify windows with per-query causal lengths; 12 and 16 rows take separate hi / lo MFMAs."""
    back = list(range(n_q - 1, -1, -1))
    check(synth.ragged_decode("iso3", "iso3", [40, 17, 1000, 2049], seed=63 + n_q, n_q=n_q, q_len_back=back,
                              n_q_heads=hq, n_kv_heads=2, head_dim=D))


@pytest.mark.parametrize("L,D", [(20000, 256), (9000, 128)])
def test_iso3_verify_window_eight_wave_shapes(L, D):
    """16 rows (separate hi / lo MFMAs) over 8 KV heads in the 8-wave launch shapes: 20,000 tokens give
    20 splits of 64 pages per KV head (160 workgroups: 64-page splits), 9,000 tokens 9 (72: 32-page
    splits)."""
    check(synth.ragged_decode("iso3", "iso3", [L], seed=68 + D, n_q=2, q_len_back=[1, 0], n_q_heads=64,
                              n_kv_heads=8, head_dim=D))


def test_iso3_decode_head_map_and_idle_kv_head():
    """An explicit head map with uneven groups; KV head 1 serves no query head."""
    w = synth.ragged_decode("iso3", "iso3", [33, 500], seed=64, n_q_heads=6, n_kv_heads=3, head_dim=128)
    check(w, head_map=[2, 0, 2, 0, 2, 2])


@pytest.mark.parametrize("lens", [[0, 5, 300], [0, 2000, 17]])
def test_iso3_decode_empty_sequence(lens):
    """A sequence with no cells gets zeros: written by its only split when the context takes one
    split (no combine launch), by the combine otherwise."""
    check(synth.ragged_decode("iso3", "iso3", lens, seed=72 + lens[1], n_q_heads=8, n_kv_heads=2, head_dim=128))


def test_iso3_decode_last_kv_head_idle():
    """The last KV head serves no query head (its workgroups find no rows)."""
    w = synth.ragged_decode("iso3", "iso3", [70, 300], seed=70, n_q_heads=4, n_kv_heads=3, head_dim=128)
    check(w, head_map=[0, 1, 0, 1])


def test_iso3_decode_mha_and_mqa():
    check(synth.ragged_decode("iso3", "iso3", [90, 260], seed=65, n_q_heads=4, n_kv_heads=4, head_dim=128))
    check(synth.ragged_decode("iso3", "iso3", [90, 260], seed=66, n_q_heads=16, n_kv_heads=1, head_dim=128))


def test_iso3_decode_batched_mixed_lengths():
    check(synth.batched_iso3_decode(seed=67, n_seqs=6, len_lo=100, len_hi=2200))


@pytest.mark.parametrize("n_q", [1, 3])
def test_iso3_decode_rising_scores_move_the_reference_max(n_q):
    """Scores that rise along the context (steadily, and with a jump of more than 2^8 in weight inside
    a page) move the lazy reference max many times, exercising the rescaling of O and l."""
    from oracle.numerics import bf16_to_f32
    L = 3000
    back = list(range(n_q - 1, -1, -1))
    w = synth.ragged_decode("iso3", "iso3", [L], seed=68 + n_q, n_q=n_q, q_len_back=back, n_q_heads=8,
                            n_kv_heads=2, head_dim=128)
    k = bf16_to_f32(w.k[0]).copy()
    q = bf16_to_f32(w.q)
    qdir = q[0, :, :4].mean(axis=(0, 1))                     # direction of KV head 0's queries
    qdir /= np.linalg.norm(qdir)
    ramp = np.linspace(0.0, 120.0, L, dtype=np.float32)
    ramp[1500:] += 80.0                                      # a jump inside page 93
    k[:, 0, :] += ramp[:, None] * qdir[None, :]
    w.k[0] = synth.bf16_bits(k)
    check(w)


def test_iso3_decode_deterministic():
    w = synth.moe_iso3_decode(ctx=5000, seed=69)
    _, a = run_decode(w)
    _, b = run_decode(w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_iso3_decode_moe_full_size_131072():
    """The ISO3 benchmark's single-sequence workload at full size, in the launch configuration the
    benchmark times."""
    check(synth.moe_iso3_decode(ctx=131072))
