"""GPU parity of decode / verify attention with an unquantised FP32 store, through the C ABI: the
single-store modes k8v32 (int8 K, FP32 V) and k32v8 (FP32 K, int8 V), and FP32 for both.

FP32 K enters the MFMAs as bf16 hi + lo parts against the exact bf16 query, FP32 V likewise against
the weights' hi + lo parts; int8 stores as in the int8 kernel.  The oracle runs fp64 attention over the
stored values.  Every case checks the slabs byte for byte against the oracle's encoding (the FP32 store
holds the bf16 inputs exactly) and the attention to max-abs 1e-3 with cosine > 0.9999 over the tensor
and every row.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, assert_slabs_equal, dev_bf16, dev_i32, gpu_append, gpu_cache,
                          oracle_decode, oracle_stores)

pytestmark = pytest.mark.gpu

MODES = [("int8", "f32"), ("f32", "int8"), ("f32", "f32")]


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
    print(f"[f32 decode] {w.fmt_k}/{w.fmt_v} {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"D={w.head_dim} n_q={w.n_q} lens={list(w.seq_lens)[:8]}", flush=True)
    cache, got = run_decode(w, head_map)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(got, oracle_decode(w, sk, sv, head_map=head_map))
    print(f"[f32 decode] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)
    return m


@pytest.mark.parametrize("fk,fv", MODES)
@pytest.mark.parametrize("D", [128, 256])
def test_f32_decode_ragged_lengths(fk, fv, D):
    """Lengths on and around page edges and a few splits deep; 4 query rows per KV head."""
    check(synth.ragged_decode(fk, fv, [1, 15, 16, 17, 300, 1024, 2100], seed=81 + D, n_q_heads=8, n_kv_heads=2,
                              head_dim=D))


@pytest.mark.parametrize("fk,fv", MODES)
@pytest.mark.parametrize("n_q,hq", [(2, 16), (3, 16), (4, 16), (3, 4)])
def test_f32_verify_windows(fk, fv, n_q, hq):
    """Verify windows with per-query causal lengths: 16, 24 and 32 rows take two row tiles."""
    back = list(range(n_q - 1, -1, -1))
    check(synth.ragged_decode(fk, fv, [40, 17, 1000, 2049], seed=83 + n_q + hq, n_q=n_q, q_len_back=back,
                              n_q_heads=hq, n_kv_heads=2, head_dim=256))


@pytest.mark.parametrize("fk,fv", MODES)
def test_f32_decode_head_map_and_idle_kv_head(fk, fv):
    """An explicit head map with uneven groups; KV head 1 serves no query head."""
    w = synth.ragged_decode(fk, fv, [33, 500], seed=84, n_q_heads=6, n_kv_heads=3, head_dim=128)
    check(w, head_map=[2, 0, 2, 0, 2, 2])


@pytest.mark.parametrize("lens", [[0, 5, 300], [0, 2000, 17]])
def test_f32_decode_empty_sequence(lens):
    """A sequence with no cells gets zeros: written by its only split when the context takes one split
    (no combine launch), by the combine otherwise."""
    check(synth.ragged_decode("int8", "f32", lens, seed=85 + lens[1], n_q_heads=8, n_kv_heads=2, head_dim=256))
    check(synth.ragged_decode("f32", "int8", lens, seed=86 + lens[1], n_q_heads=8, n_kv_heads=2, head_dim=256))


def test_f32_decode_mha_and_mqa():
    check(synth.ragged_decode("int8", "f32", [90, 260], seed=87, n_q_heads=4, n_kv_heads=4, head_dim=128))
    check(synth.ragged_decode("f32", "int8", [90, 260], seed=88, n_q_heads=16, n_kv_heads=1, head_dim=128))


@pytest.mark.parametrize("fk,fv", MODES)
def test_f32_decode_wide_value_range(fk, fv):
    """K and V far from unit scale (x 3e4 and x 1e-4): the hi / lo parts keep 16 significant bits at
    any magnitude; compared relative to the output's magnitude."""
    from oracle.numerics import bf16_to_f32
    w = synth.ragged_decode(fk, fv, [700, 33, 4000], seed=89, n_q=2, q_len_back=[1, 0], n_q_heads=8, n_kv_heads=2,
                            head_dim=256)
    for b in range(w.batch):
        w.k[b] = synth.bf16_bits(bf16_to_f32(w.k[b]) * np.float32(1.0e-4))
        w.v[b] = synth.bf16_bits(bf16_to_f32(w.v[b]) * np.float32(3.0e4))
    w.q = synth.bf16_bits(bf16_to_f32(w.q) * np.float32(3.0e4))
    cache, got = run_decode(w)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    ref = oracle_decode(w, sk, sv)
    scale = float(np.max(np.abs(ref)))
    assert_attention_close(got / scale, ref / scale)


@pytest.mark.parametrize("n_q", [1, 3])
def test_f32_decode_rising_scores_move_the_reference_max(n_q):
    """Scores that rise along the context (steadily, and with a jump inside a page) move the lazy
    reference max many times, exercising the rescaling of O, l and the int8 V weight sums."""
    from oracle.numerics import bf16_to_f32
    L = 3000
    back = list(range(n_q - 1, -1, -1))
    for fk, fv in MODES[:2]:
        w = synth.ragged_decode(fk, fv, [L], seed=90 + n_q, n_q=n_q, q_len_back=back, n_q_heads=8, n_kv_heads=2,
                                head_dim=256)
        k = bf16_to_f32(w.k[0]).copy()
        q = bf16_to_f32(w.q)
        qdir = q[0, :, :4].mean(axis=(0, 1))
        qdir /= np.linalg.norm(qdir)
        ramp = np.linspace(0.0, 120.0, L, dtype=np.float32)
        ramp[1500:] += 80.0
        k[:, 0, :] += ramp[:, None] * qdir[None, :]
        w.k[0] = synth.bf16_bits(k)
        check(w)


def test_f32_decode_deterministic():
    w = synth.moe_single_store_decode("f32", "int8", ctx=5000)
    _, a = run_decode(w)
    _, b = run_decode(w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fk,fv", MODES[:2])
def test_f32_decode_moe_full_size_131072(fk, fv):
    """The single-store benchmark workloads at full size, in the launch configuration the benchmark
    times."""
    check(synth.moe_single_store_decode(fk, fv, ctx=131072))
