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
from oracle import attention as oatt
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
    make three row-group workgroups per split, each of which encodes and stores the window's cells
    of its split (identical bytes) before reading them back."""
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


@pytest.mark.parametrize("fk,fv,D,n_q", [("int8", "int8", 256, 1), ("int8", "int8", 256, 3), ("int8", "q4h", 256, 3),
                                         ("int8", "f32", 128, 3)])
def test_fused_short_sequences_skip_missing_positions(fk, fv, D, n_q):
    """A sequence shorter than the step's window (an idle slot of length 0, or 2 cells under a 3-token
    window) has no cell for the window's first tokens: they are skipped, never written elsewhere.  A
    zero-length sequence's page-table row reads page 0, which holds another sequence's cells: every
    cell of the cache must stay exactly as the oracle encodes the sequences' real tokens, and the
    short sequence's cells hold its own last tokens."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    lens = [0, 300, 2, 17] if n_q == 3 else [0, 300, 17]
    back = list(range(n_q - 1, -1, -1)) if n_q > 1 else None
    w = synth.ragged_decode(fk, fv, lens, seed=70 + n_q + D, n_q=n_q, n_q_heads=16, n_kv_heads=2, head_dim=D,
                            q_len_back=back)
    assert int(w.block_table[0, 0]) == 0, "the zero-length row points at page 0"
    rng = np.random.default_rng(71)
    junk = synth.normal_bf16(rng, (w.n_kv_heads, D))          # tokens with no cell: must go nowhere
    kn = np.stack([np.stack([w.k[b][L - n_q + t] if L - n_q + t >= 0 else junk for t in range(n_q)])
                   for b, L in enumerate(lens)])
    vn = np.stack([np.stack([w.v[b][L - n_q + t] if L - n_q + t >= 0 else junk for t in range(n_q)])
                   for b, L in enumerate(lens)])
    cache, pages = gpu_cache(w)
    seq = np.concatenate([np.full(max(L - n_q, 0), b, np.int32) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(max(L - n_q, 0), dtype=np.int32) for L in lens])
    kp = np.concatenate([w.k[b][:max(L - n_q, 0)] for b, L in enumerate(lens)])
    vp = np.concatenate([w.v[b][:max(L - n_q, 0)] for b, L in enumerate(lens)])
    kvq.kvq_append(cache, pages, dev_bf16(kp), dev_bf16(vp), dev_i32(seq), dev_i32(pos))
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn_append(cache, pages, dev_bf16(kn), dev_bf16(vn), dev_bf16(w.q), q_lens=q_lens,
                                     sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    sk, sv = oracle_stores(w)                                 # every real token of every sequence, nothing else
    assert_slabs_equal(cache, sk, sv)
    got = out.cpu().numpy()
    assert_attention_close(got, oracle_decode(w, sk, sv))
    assert not got[0].any(), "the zero-length sequence's rows are zeros"


def test_fused_moe_full_size_131072():
    """The benchmark's workload and launch configuration at full size."""
    m = check_fused(synth.moe_int8_decode(ctx=131072))
    print(f"[fused 131072] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


def test_fused_moe_full_size_65536():
    """The MoE layer at 65,536 tokens (the 64K column of strata PR #2698, Measurements): a launch plan
    with 32-page splits, at full size in the fused launch configuration."""
    m = check_fused(synth.moe_int8_decode(ctx=65536))
    print(f"[fused 65536] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}")


def test_fused_batched_full_size_all_sequences():
    """The 32-sequence batched workload (4,096-32,768 tokens each, 32 / 8 heads, head_dim 128) at full
    size in the benchmark's launch configuration (fused quantize-on-write + decode).  The oracle runs
    one sequence at a time (its own pages only, so host memory stays bounded): every cell of every
    sequence -- the prefix written by kvq_append and the step's cell written by the decode launch -- is
    compared byte for byte in both stores (codes and scales), and every output row to the tolerance;
    the fused output equals append + decode bit for bit over the whole batch."""
    from oracle import paged as opaged
    from kvq_testutil import tile_index
    w = synth.batched_int8_decode()
    lens = np.asarray(w.seq_lens)
    print(f"[fused batched] {w.batch} sequences, {int(lens.sum())} cells", flush=True)
    cache, got = run_fused(w)
    slabs = {x: (getattr(cache, f"{x}_codes").cpu().numpy(), getattr(cache, f"{x}_scales").cpu().numpy())
             for x in ("k", "v")}
    idx = {"k": tile_index("k_chunk", w.head_dim), "v": tile_index("v_quad", w.head_dim)}
    worst = [0.0, 1.0, 1.0]
    for b in range(w.batch):
        L = int(lens[b])
        need = (L + w.page_size - 1) // w.page_size
        bt = np.arange(need, dtype=np.int32)[None, :]             # the sequence's pages, renumbered
        st = {x: opaged.Store.empty(getattr(w, f"fmt_{x}"), need, w.n_kv_heads, w.page_size, w.head_dim)
              for x in ("k", "v")}
        opaged.append(st["k"], bt, np.zeros(L, int), np.arange(L), w.k[b], w.page_size)
        opaged.append(st["v"], bt, np.zeros(L, int), np.arange(L), w.v[b], w.page_size)
        pages = w.block_table[b, :need]
        for x in ("k", "v"):
            codes = slabs[x][0][pages][:, :, idx[x]]                  # [need][hkv][slot][code byte]
            assert np.array_equal(codes, st[x].codes), f"{x} codes of sequence {b} (length {L})"
            assert np.array_equal(slabs[x][1][pages].view(np.uint16), st[x].scales.view(np.uint16)), \
                f"{x} scales of sequence {b}"
        ref = oatt.decode(st["k"], st["v"], bt, np.array([L], np.int32), w.q[b:b + 1], w.page_size, w.sm_scale)
        m = assert_attention_close(got[b:b + 1], ref)
        worst = [max(worst[0], m[0]), min(worst[1], m[1]), min(worst[2], m[2])]
    print(f"[fused batched] all {w.batch} sequences: max-abs {worst[0]:.2e} min cosine {worst[1]:.8f} "
          f"min row cosine {worst[2]:.8f}")
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
