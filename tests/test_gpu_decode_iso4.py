"""GPU parity of the ISO4 store (append, gather) and of decode / verify attention over ISO4 K and V,
through the C ABI.

ISO4 runs through the ISO3 attention kernel with 4-bit codes: a 256-entry table of fp16 level pairs
indexed by one code byte, binary32 norms.  Every case checks the slabs byte for byte against the
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
    return cache, pages, out.cpu().numpy()


def check(w, head_map=None):
    print(f"[iso4 decode] {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} n_q={w.n_q} "
          f"lens={list(w.seq_lens)[:8]}", flush=True)
    cache, _, got = run_decode(w, head_map)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(got, oracle_decode(w, sk, sv, head_map=head_map))
    print(f"[iso4 decode] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)
    return m


@pytest.mark.parametrize("D", [128, 256, 512])
def test_iso4_append_and_gather_bitexact(D):
    """Encoder bytes and norms equal the oracle's; the gather's F32 output equals the oracle's
    dequantisation bit for bit, F16 / BF16 its rounding."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    from oracle import paged as opaged
    w = synth.ragged_decode("iso4", "iso4", [77, 33], head_dim=D, seed=91 + D, n_q_heads=2, n_kv_heads=2)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    for which, st in (("k", sk), ("v", sv)):
        for seq, start, count in ((0, 0, 77), (0, 13, 40), (1, 31, 2)):
            got = kvq.kvq_dequant_gather(cache, pages, which, seq, start, count, "f32").cpu().numpy()
            ref = opaged.gather(st, w.block_table, seq, start, count, 16, quat=w.quat)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{which} seq {seq} [{start},+{count})"
            lowp = kvq.kvq_dequant_gather(cache, pages, which, seq, start, count, "bf16")
            assert torch.equal(lowp, torch.from_numpy(ref).to(torch.bfloat16).cuda())


@pytest.mark.parametrize("D", [128, 256])
def test_iso4_decode_ragged_lengths(D):
    check(synth.ragged_decode("iso4", "iso4", [1, 15, 16, 17, 300, 1024, 2100], seed=92 + D, n_q_heads=8,
                              n_kv_heads=2, head_dim=D))


@pytest.mark.parametrize("D", [128, 256])
def test_iso4_decode_64_page_splits(D):
    """Four sequences over eight KV heads: 9 x 8 x 4 = 288 splits of 64 pages fill more than one
    workgroup per CU, so the plan keeps 64-page splits (the other launch shape: 4 waves x 16 pages)."""
    check(synth.ragged_decode("iso4", "iso4", [9000, 8200, 4100, 9000], seed=83, n_q_heads=16, n_kv_heads=8,
                              head_dim=D))


def test_iso4_decode_eight_rows_head_dim_256():
    check(synth.ragged_decode("iso4", "iso4", [5, 700, 4100], seed=93, n_q_heads=16, n_kv_heads=2, head_dim=256))


@pytest.mark.parametrize("n_q,hq,D", [(3, 8, 128), (2, 16, 256), (2, 4, 128)])
def test_iso4_verify_windows(n_q, hq, D):
    back = list(range(n_q - 1, -1, -1))
    check(synth.ragged_decode("iso4", "iso4", [40, 17, 1000, 2049], seed=94 + n_q, n_q=n_q, q_len_back=back,
                              n_q_heads=hq, n_kv_heads=2, head_dim=D))


@pytest.mark.parametrize("L,D", [(20000, 128), (9000, 256)])
def test_iso4_verify_window_eight_wave_shapes(L, D):
    """16 rows over 8 KV heads in the 8-wave launch shapes (64-page and 32-page splits)."""
    check(synth.ragged_decode("iso4", "iso4", [L], seed=97 + D, n_q=2, q_len_back=[1, 0], n_q_heads=64,
                              n_kv_heads=8, head_dim=D))


def test_iso4_decode_head_map_and_idle_kv_head():
    w = synth.ragged_decode("iso4", "iso4", [33, 500], seed=95, n_q_heads=6, n_kv_heads=3, head_dim=128)
    check(w, head_map=[2, 0, 2, 0, 2, 2])


@pytest.mark.parametrize("lens", [[0, 5, 300], [0, 2000, 17]])
def test_iso4_decode_empty_sequence(lens):
    check(synth.ragged_decode("iso4", "iso4", lens, seed=96 + lens[1], n_q_heads=8, n_kv_heads=2, head_dim=128))


def test_iso4_decode_mha_and_mqa():
    check(synth.ragged_decode("iso4", "iso4", [90, 260], seed=97, n_q_heads=4, n_kv_heads=4, head_dim=128))
    check(synth.ragged_decode("iso4", "iso4", [90, 260], seed=98, n_q_heads=16, n_kv_heads=1, head_dim=128))


def test_iso4_decode_rising_scores_move_the_reference_max():
    from oracle.numerics import bf16_to_f32
    L = 3000
    w = synth.ragged_decode("iso4", "iso4", [L], seed=99, n_q=3, q_len_back=[2, 1, 0], n_q_heads=8, n_kv_heads=2,
                            head_dim=128)
    k = bf16_to_f32(w.k[0]).copy()
    q = bf16_to_f32(w.q)
    qdir = q[0, :, :4].mean(axis=(0, 1))
    qdir /= np.linalg.norm(qdir)
    ramp = np.linspace(0.0, 120.0, L, dtype=np.float32)
    ramp[1500:] += 80.0
    k[:, 0, :] += ramp[:, None] * qdir[None, :]
    w.k[0] = synth.bf16_bits(k)
    check(w)


def test_iso4_decode_moe_full_size_131072():
    """The ISO4 benchmark's single-sequence workload at full size, in the launch configuration the
    benchmark times."""
    check(synth.moe_iso3_decode(ctx=131072, fmt="iso4"))
