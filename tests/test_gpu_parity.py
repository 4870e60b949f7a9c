"""GPU parity: the HIP path through the C ABI against the oracle on the same seeded inputs.

Codes, scales and norms must be byte-identical for every cell (and untouched cells must stay
zero); gather F32 output must be bit-exact; attention must be within max-abs 1e-3 with cosine
> 0.9999 over the whole output and over every row.
"""
import numpy as np
import pytest

import synth
from oracle import paged as opaged
from oracle.numerics import bf16_to_f32
from kvq_testutil import (assert_attention_close, assert_slabs_equal, gpu_append, gpu_cache, oracle_decode,
                          oracle_stores)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_paged_kv_kvq_amd as kvq
    kvq.lib()


def run_decode(w, head_map=None):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    from kvq_testutil import dev_bf16, dev_i32
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q = dev_bf16(w.q)
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn(cache, pages, q, q_lens=q_lens, head_map=head_map, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return cache, pages, out.cpu().numpy()


def check_decode(w, head_map=None):
    print(f"[decode parity] {w.name} fmt={w.fmt_k}/{w.fmt_v} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"D={w.head_dim} n_q={w.n_q} lens={list(w.seq_lens)[:8]}", flush=True)
    cache, pages, got = run_decode(w, head_map)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    ref = oracle_decode(w, sk, sv, head_map=head_map)
    return assert_attention_close(got, ref)


# ---------------------------------------------------------------------------------------------
# quantize-on-write and gather

@pytest.mark.parametrize("fmt_k,fmt_v,D", [("int8", "int8", 128), ("int8", "int8", 256), ("int8", "int8", 64),
                                           ("int8", "q4h", 256), ("q4h", "q4h", 256), ("iso3", "iso3", 128),
                                           ("iso3", "iso3", 256)])
def test_append_bitexact_through_random_pages(fmt_k, fmt_v, D):
    w = synth.ragged_decode(fmt_k, fmt_v, [37, 64, 5, 1, 130], head_dim=D, seed=21, n_q_heads=4, n_kv_heads=2)
    print(f"[append] {fmt_k}/{fmt_v} D={D}", flush=True)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    import torch
    torch.cuda.synchronize()
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


def test_append_special_values():
    """All-zero groups, exact ties and a lone non-zero value go through the same rules as the oracle."""
    w = synth.ragged_decode("int8", "q4h", [16], head_dim=256, seed=22, n_q_heads=2, n_kv_heads=1)
    k = bf16_to_f32(w.k[0]).copy()
    k[0] = 0.0                                    # all-zero cell
    k[1, 0, :64] = 0.0                            # one zero group
    k[2, 0, :] = np.float32(0.5)                  # equal values
    k[3, 0, :64] = 0.0
    k[3, 0, 5] = -3.0                             # lone value
    k[4, 0, :8] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5]   # scale 1, ties to even
    w.k[0] = synth.bf16_bits(k)
    v = bf16_to_f32(w.v[0]).copy()
    v[0] = 0.0
    v[1, 0, :] = 1.0                              # rotates onto one coordinate
    w.v[0] = synth.bf16_bits(v)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    import torch
    torch.cuda.synchronize()
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


@pytest.mark.parametrize("fmt,D,fk", [("int8", 128, None), ("int8", 256, None), ("q4h", 256, "int8"), ("q4h", 256, "q4h"),
                                      ("iso3", 128, None), ("iso3", 256, None), ("f32", 256, None),
                                      ("f32", 128, "int8"), ("int8", 256, "f32")])
def test_gather_bitexact(fmt, D, fk):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    fk = fk or fmt
    w = synth.ragged_decode(fk, fmt, [77, 33], head_dim=D, seed=23, n_q_heads=2, n_kv_heads=2)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    sk, sv = oracle_stores(w)
    for which, st in (("k", sk), ("v", sv)):
        for seq, start, count in ((0, 0, 77), (0, 13, 40), (1, 31, 2), (1, 0, 0)):
            got = kvq.kvq_dequant_gather(cache, pages, which, seq, start, count, "f32").cpu().numpy()
            ref = opaged.gather(st, w.block_table, seq, start, count, 16, quat=w.quat, rotated=True)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{which} seq {seq} [{start},+{count})"
            for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
                lowp = kvq.kvq_dequant_gather(cache, pages, which, seq, start, count, dt)
                exp = torch.from_numpy(ref).to(tdt).cuda()
                assert torch.equal(lowp, exp), f"{which} {dt} rounding"
            if st.fmt == "q4h" and count:
                un = kvq.kvq_dequant_gather(cache, pages, which, seq, start, count, "f32", unrotate=True).cpu().numpy()
                ref64 = opaged.gather(st, w.block_table, seq, start, count, 16, rotated=False)
                assert np.max(np.abs(un - ref64)) <= 2e-6 * max(1.0, np.max(np.abs(ref64)))


# ---------------------------------------------------------------------------------------------
# decode / verify attention

def test_decode_tiny_int8_full_size():
    check_decode(synth.tiny_int8_decode())


@pytest.mark.parametrize("ctx", [1, 15, 16, 17, 700, 3001])
def test_decode_moe_shape_ragged(ctx):
    check_decode(synth.moe_int8_decode(ctx=ctx, seed=100 + ctx))


def test_decode_batched_mixed_lengths():
    w = synth.batched_int8_decode(seed=31, n_seqs=6, len_lo=100, len_hi=2200)
    check_decode(w)


def test_decode_edge_lengths_and_head_map():
    w = synth.ragged_decode("int8", "int8", [0, 1, 15, 16, 17, 300, 1024], seed=32, n_q_heads=6, n_kv_heads=3,
                            head_dim=64)
    hm = [2, 0, 1, 0, 2, 2]                       # uneven, non-contiguous query-head groups
    check_decode(w, head_map=hm)


@pytest.mark.parametrize("fmt_v", ["int8", "q4h"])
def test_decode_empty_sequence_multi_split(fmt_v):
    """An empty sequence next to one that takes several splits: its zeros come from the combine."""
    check_decode(synth.ragged_decode("int8", fmt_v, [0, 2000, 17], seed=73, n_q_heads=8, n_kv_heads=2,
                                     head_dim=256))


def test_decode_last_kv_head_idle():
    """The last KV head serves no query head (its workgroups find no rows)."""
    w = synth.ragged_decode("int8", "int8", [70, 300], seed=71, n_q_heads=4, n_kv_heads=3, head_dim=128)
    check_decode(w, head_map=[0, 1, 0, 1])


def test_decode_mha_and_mqa():
    check_decode(synth.ragged_decode("int8", "int8", [200, 45], seed=33, n_q_heads=4, n_kv_heads=4, head_dim=128))
    check_decode(synth.ragged_decode("int8", "int8", [513], seed=34, n_q_heads=16, n_kv_heads=1, head_dim=128))


def test_verify_int8_multi_query():
    w = synth.ragged_decode("int8", "int8", [900, 47, 300], seed=35, n_q=4, q_len_back=[3, 2, 1, 0], n_q_heads=8,
                            n_kv_heads=2, head_dim=128)
    check_decode(w)


def test_verify_k8v4_scaled():
    check_decode(synth.k8v4_verify(ctx=2500, seed=36))


@pytest.mark.parametrize("n_q,hq,hkv", [(2, 16, 2), (3, 8, 2), (4, 16, 2), (1, 12, 1)])
def test_verify_k8v4_row_tiles(n_q, hq, hkv):
    """k8v4 with more than 8 rows per KV head: one workgroup per split holds all rows in row tiles
    of 16 (16, 12, 32 and 12 rows), V entering the MFMA as code x scale / 16 in two fp16 parts."""
    back = list(range(n_q - 1, -1, -1))
    w = synth.ragged_decode("int8", "q4h", [700, 33, 4000], seed=60 + n_q + hq, n_q=n_q, q_len_back=back,
                            n_q_heads=hq, n_kv_heads=hkv, head_dim=256)
    check_decode(w)


@pytest.mark.parametrize("v_mul", [2.0e4, 1.0e-5])
def test_verify_k8v4_row_tiles_value_range(v_mul):
    """V far from unit scale through the row-tile kernel's fp16 V parts: scales near the top of fp16
    (products up to 8 x d / 16) and scales so small the products are subnormal in fp16."""
    w = synth.ragged_decode("int8", "q4h", [700, 33, 4000], seed=66, n_q=3, q_len_back=[2, 1, 0], n_q_heads=8,
                            n_kv_heads=2, head_dim=256)
    for b in range(w.batch):
        w.v[b] = synth.bf16_bits(bf16_to_f32(w.v[b]) * np.float32(v_mul))
    cache, pages, got = run_decode(w)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    ref = oracle_decode(w, sk, sv)
    scale = float(np.max(np.abs(ref)))
    # the bound is relative to the output's magnitude (max-abs 1e-3 at unit scale)
    assert_attention_close(got / scale, ref / scale)


def test_decode_k8v4_single_query():
    check_decode(synth.ragged_decode("int8", "q4h", [1000, 33], seed=37, n_q_heads=16, n_kv_heads=2, head_dim=256))


def test_decode_outlier_peaked_attention():
    """A query aligned with one key's outlier channels makes attention nearly one-hot."""
    w = synth.moe_int8_decode(ctx=4000, seed=38)
    k = bf16_to_f32(w.k[0])
    q = bf16_to_f32(w.q).copy()
    q[0, 0, :8] = k[1234, 0] * 4.0                # heads of KV head 0 look at key 1234
    w.q = synth.bf16_bits(q)
    check_decode(w)


@pytest.mark.parametrize("fmt_v,n_q", [("int8", 1), ("q4h", 3)])
def test_decode_rising_scores_move_the_reference_max(fmt_v, n_q):
    """Scores that rise along the context (steadily, and with jumps of more than 2^8 in weight
    inside a page) make the softmax reference max move many times: exercises the rescaling of O
    and l that is skipped while scores stay within 2^8 of the reference."""
    L = 3000
    w = synth.ragged_decode("int8", fmt_v, [L], seed=40 + n_q, n_q=n_q, n_q_heads=16, n_kv_heads=2, head_dim=256)
    k = bf16_to_f32(w.k[0]).copy()
    q = bf16_to_f32(w.q)
    qdir = q[0, :, :8].mean(axis=(0, 1))                     # direction of KV head 0's queries
    qdir /= np.linalg.norm(qdir)
    ramp = np.linspace(0.0, 120.0, L, dtype=np.float32)
    ramp[1500:] += 80.0                                      # a jump inside page 93
    k[:, 0, :] += ramp[:, None] * qdir[None, :]
    w.k[0] = synth.bf16_bits(k)
    check_decode(w)


def test_decode_deterministic():
    w = synth.moe_int8_decode(ctx=5000, seed=39)
    _, _, a = run_decode(w)
    _, _, b = run_decode(w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_decode_moe_full_size_131072():
    """The benchmark's workload and launch configuration at full size."""
    m = check_decode(synth.moe_int8_decode(ctx=131072))
    print(f"[131072] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


def test_decode_moe_full_size_65536():
    """The MoE layer at 65,536 tokens (the 64K column of strata PR #2698, Measurements), whose launch
    plan takes 32-page splits, at full size."""
    m = check_decode(synth.moe_int8_decode(ctx=65536))
    print(f"[65536] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


def test_verify_k8v4_full_size():
    m = check_decode(synth.k8v4_verify())
    print(f"[k8v4 118750] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")
