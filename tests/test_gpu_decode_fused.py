"""GPU parity of the fused decode step (kvq_decode_attn_append: quantize-on-write of the step's
tokens and decode attention in one launch sequence), through the C ABI, for int8 K and V, the k8v4
hybrid (q4_0 V encoded by one wave per cell) and the single-store modes (int8 / FP32 stores).

Every case checks the slabs byte for byte against the oracle's encoding of every token (prefix
and step), the attention against the oracle (max-abs 1e-3, cosine > 0.9999 over the tensor and
every row), and that the output is bit-identical to kvq_append followed by kvq_decode_attn.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, assert_slabs_equal, dev_bf16, dev_i32, gpu_append, gpu_cache,
                          oracle_decode, oracle_stores)

pytestmark = pytest.mark.gpu


def step_tokens(w):
    """The step's new K and V as bf16 [batch][n_q][n_kv_heads][head_dim] (the last n_q cells)."""
    assert w.n_step == w.n_q, "the fused step appends one token per query token"
    ks = np.stack([w.k[b][int(w.seq_lens[b]) - w.n_q:int(w.seq_lens[b])] for b in range(w.batch)])
    vs = np.stack([w.v[b][int(w.seq_lens[b]) - w.n_q:int(w.seq_lens[b])] for b in range(w.batch)])
    return ks, vs


def run_fused(w, head_map=None):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    ks, vs = step_tokens(w)
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn_append(cache, pages, dev_bf16(ks), dev_bf16(vs), dev_bf16(w.q), q_lens=q_lens,
                                     head_map=head_map, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return cache, out.cpu().numpy()


def run_unfused(w, head_map=None):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn(cache, pages, dev_bf16(w.q), q_lens=q_lens, head_map=head_map, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_fused(w, head_map=None):
    print(f"[fused decode] {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} D={w.head_dim} n_q={w.n_q} "
          f"lens={list(w.seq_lens)[:8]}", flush=True)
    cache, got = run_fused(w, head_map)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(got, oracle_decode(w, sk, sv, head_map=head_map))
    ref = run_unfused(w, head_map)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "fused and unfused outputs differ"
    return m


@pytest.mark.parametrize("ctx", [1, 15, 16, 17, 700, 3001])
def test_fused_moe_shape_ragged(ctx):
    """The new cell in page 0 (patched before the first page is processed), on page edges, and deep
    in a split."""
    check_fused(synth.moe_int8_decode(ctx=ctx, seed=200 + ctx))


def test_fused_batched_mixed_lengths():
    check_fused(synth.batched_int8_decode(seed=51, n_seqs=6, len_lo=100, len_hi=2200))


def test_fused_edge_lengths_and_head_map():
    w = synth.ragged_decode("int8", "int8", [1, 15, 16, 17, 300, 1024], seed=52, n_q_heads=6, n_kv_heads=3,
                            head_dim=64)
    check_fused(w, head_map=[2, 0, 1, 0, 2, 2])


def test_fused_kv_head_without_queries_still_appends():
    """KV head 1 serves no query head: its workgroups attend nothing but must still write the cell."""
    w = synth.ragged_decode("int8", "int8", [40, 200], seed=53, n_q_heads=4, n_kv_heads=3, head_dim=128)
    check_fused(w, head_map=[0, 0, 2, 2])


@pytest.mark.parametrize("lens", [[3, 17, 33, 100], [18, 16, 1000, 64]])
def test_fused_verify_window_across_page_edges(lens):
    """Three new tokens per sequence, some windows straddling a page boundary; 24 rows per KV head
    make three row-group workgroups per split (all patch, one stores)."""
    w = synth.ragged_decode("int8", "int8", lens, seed=54 + lens[0], n_q=3, q_len_back=[2, 1, 0], n_q_heads=16,
                            n_kv_heads=2, head_dim=256)
    check_fused(w)


def test_fused_four_queries_head_dim_128():
    w = synth.ragged_decode("int8", "int8", [900, 47, 300], seed=55, n_q=4, q_len_back=[3, 2, 1, 0], n_q_heads=8,
                            n_kv_heads=2, head_dim=128)
    check_fused(w)


def test_fused_graph_replays():
    """Captured in a HIP graph and replayed several times with eager work between the replays: every
    replay gives the eager output, and the slabs stay the oracle's (rewriting a cell is idempotent)."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_decode("int8", "int8", [4096, 300], seed=56, n_q_heads=16, n_kv_heads=2, head_dim=256)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    ks, vs = step_tokens(w)
    kn, vn, q = dev_bf16(ks), dev_bf16(vs), dev_bf16(w.q)
    out = torch.empty((w.batch, w.n_q, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nbytes = kvq.kvq_decode_workspace_bytes(cache, pages.batch, pages.max_pages, w.n_q, w.n_q_heads)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step_fn():
        kvq.kvq_decode_attn_append(cache, pages, kn, vn, q, sm_scale=w.sm_scale, out=out, workspace=ws)

    step_fn()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn()
    for r in range(4):
        out.zero_()
        scratch = torch.randn(1 << 20, device="cuda").sum()       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        assert torch.isfinite(scratch)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    assert_attention_close(eager.cpu().numpy(), oracle_decode(w, sk, sv))


def test_fused_moe_full_size_131072():
    """The benchmark's workload and launch configuration at full size."""
    m = check_fused(synth.moe_int8_decode(ctx=131072))
    print(f"[fused 131072] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


def test_fused_batched_full_size_sampled_sequences():
    """The 32-sequence batched workload (4,096-32,768 tokens each, 32 / 8 heads, head_dim 128) at full
    size in the benchmark's launch configuration (fused quantize-on-write + decode).  The oracle encodes
    and attends a sample of sequences (shortest, longest, first, last); their step cells are compared
    byte for byte and their outputs to the tolerance; the fused output equals append + decode bit for
    bit over the whole batch."""
    from oracle import paged as opaged
    w = synth.batched_int8_decode()
    lens = np.asarray(w.seq_lens)
    seqs = sorted({0, w.batch - 1, int(np.argmin(lens)), int(np.argmax(lens))})
    print(f"[fused batched] sampled sequences {seqs} of {w.batch}, lengths {[int(lens[b]) for b in seqs]}", flush=True)
    cache, got = run_fused(w)
    sk = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = opaged.Store.empty(w.fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    for b in seqs:
        L = int(lens[b])
        opaged.append(sk, w.block_table, np.full(L, b), np.arange(L), w.k[b], w.page_size)
        opaged.append(sv, w.block_table, np.full(L, b), np.arange(L), w.v[b], w.page_size)
    ref = oracle_decode(w, sk, sv, seqs=seqs)
    assert_attention_close(got[seqs], ref[seqs])
    kc, ks = (cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy())
    for b in seqs:                                   # the step's cell (last position) of each sampled sequence
        pos = int(lens[b]) - 1
        page, slot = int(w.block_table[b, pos // 16]), pos % 16
        from kvq_testutil import tile_index
        idx = tile_index("k_chunk", w.head_dim)[slot]
        assert np.array_equal(kc[page][:, idx], sk.codes[page, :, slot, :]), f"K cell of sequence {b}"
        assert np.array_equal(ks[page][:, slot].view(np.uint16), sk.scales[page, :, slot].view(np.uint16))
    assert np.array_equal(got.view(np.uint32), run_unfused(w).view(np.uint32)), "fused and unfused outputs differ"

@pytest.mark.parametrize("lens", [[33, 2500], [16, 17, 1000]])
def test_fused_k8v4_single_query(lens):
    """int8 K + Hadamard-rotated q4_0 V, one query token, 8 rows per KV head (duplicated columns)."""
    check_fused(synth.ragged_decode("int8", "q4h", lens, seed=55 + len(lens), n_q_heads=16, n_kv_heads=2,
                                    head_dim=256))


@pytest.mark.parametrize("ctx", [3, 17, 2500])
def test_fused_k8v4_verify_windows(ctx):
    """k8v4 MTP verify (3 tokens, 24 rows in two row tiles) with the window's cells written by the launch,
    on and across page edges."""
    check_fused(synth.k8v4_verify(ctx=ctx, seed=56 + ctx))


def test_fused_k8v4_small_new_v_scale():
    """The row-tile kernel's fp16 V parts need every V d of a wave's pages >= 2^-10: a window whose new
    V tokens are tiny (d far below that) while the cache holds ordinary values must take the bf16
    parts, decided from the encoder's d (the scale scan may read the slot as it was before the store)."""
    from oracle.numerics import bf16_to_f32
    w = synth.k8v4_verify(ctx=700, seed=57)
    v = bf16_to_f32(w.v[0]).copy()
    v[-3:] *= np.float32(1e-5)
    w.v[0] = synth.bf16_bits(v)
    check_fused(w)


def test_fused_k8v4_full_size_118750():
    """The k8v4 verify workload at full size in the fused launch configuration."""
    m = check_fused(synth.k8v4_verify())
    print(f"[fused k8v4 118750] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


@pytest.mark.parametrize("fk,fv", [("int8", "f32"), ("f32", "int8"), ("f32", "f32")])
@pytest.mark.parametrize("D", [128, 256])
def test_fused_single_store_modes(fk, fv, D):
    """k8v32 / k32v8 / FP32: the step's cells written by the decode launch (int8 encoded or FP32 values),
    one query token and a verify window across page edges; a KV head without queries still appends."""
    check_fused(synth.ragged_decode(fk, fv, [1, 17, 300, 2100], seed=60 + D, n_q_heads=8, n_kv_heads=2,
                                    head_dim=D))
    check_fused(synth.ragged_decode(fk, fv, [3, 16, 18, 1000], seed=61 + D, n_q=3, q_len_back=[2, 1, 0],
                                    n_q_heads=16, n_kv_heads=2, head_dim=D))
    w = synth.ragged_decode(fk, fv, [40, 300], seed=62 + D, n_q_heads=4, n_kv_heads=3, head_dim=D)
    check_fused(w, head_map=[0, 2, 0, 2])


def test_fused_k8v32_full_size_131072():
    """The k8v32 workload at full size in the fused launch configuration."""
    m = check_fused(synth.moe_single_store_decode("int8", "f32", ctx=131072))
    print(f"[fused k8v32 131072] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")
