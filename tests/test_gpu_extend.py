"""GPU parity of extend (prefill chunk) attention over ISO3- and int8-packed prefixes, through the C ABI.

Each case fills the cache with the prefix through kvq_append, runs kvq_extend_attn on the chunk's
bf16 tokens (deferred packing on), and compares with the oracle: attention element by element
(max-abs 1e-3, cosine > 0.9999 over the tensor and every row), and the slabs after packing byte
for byte with the oracle's encoding of every token.
"""
import numpy as np
import pytest

import synth
from oracle import attention as oatt
from oracle import paged as opaged
from kvq_testutil import assert_attention_close, assert_slabs_equal, dev_bf16, dev_i32, oracle_stores

pytestmark = pytest.mark.gpu


def chunk_inputs(w):
    """(prefix lens, cu_new, new K bf16, new V bf16) of an extend workload."""
    pre, new = w.prefix_lens(), w.new_lens()
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    kn = [w.k[b][int(pre[b]):] for b in range(w.batch)]
    vn = [w.v[b][int(pre[b]):] for b in range(w.batch)]
    shape = (0, w.n_kv_heads, w.head_dim)
    cat = lambda xs: np.concatenate(xs) if sum(len(x) for x in xs) else np.zeros(shape, np.uint16)
    return pre, cu, cat(kn), cat(vn)


def oracle_prefix_stores(w):
    pre = w.prefix_lens()
    sk = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = opaged.Store.empty(w.fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    for b in range(w.batch):
        P = int(pre[b])
        if P:
            opaged.append(sk, w.block_table, np.full(P, b), np.arange(P), w.k[b][:P], w.page_size, quat=w.quat)
            opaged.append(sv, w.block_table, np.full(P, b), np.arange(P), w.v[b][:P], w.page_size, quat=w.quat)
    return sk, sv


def run_extend(w, head_map=None, pack_after=True):
    """Fill the prefix, run extend on the GPU.  Returns (cache, out as numpy)."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    pre, cu, kn, vn = chunk_inputs(w)
    cache = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
    pages = kvq.Pages(dev_i32(w.block_table), dev_i32(pre))
    seqs = [np.full(int(pre[b]), b, np.int32) for b in range(w.batch)]
    if int(pre.sum()):
        tok_seq = np.concatenate(seqs)
        tok_pos = np.concatenate([np.arange(int(pre[b]), dtype=np.int32) for b in range(w.batch)])
        kp = np.concatenate([w.k[b][:int(pre[b])] for b in range(w.batch)])
        vp = np.concatenate([w.v[b][:int(pre[b])] for b in range(w.batch)])
        kvq.kvq_append(cache, pages, dev_bf16(kp), dev_bf16(vp), dev_i32(tok_seq), dev_i32(tok_pos))
    max_new = int(w.new_lens().max()) if w.batch else 0
    out = kvq.kvq_extend_attn(cache, pages, dev_bf16(w.q), dev_bf16(kn), dev_bf16(vn), dev_i32(cu), max_new,
                              head_map=head_map, sm_scale=w.sm_scale, pack_after=pack_after)
    torch.cuda.synchronize()
    return cache, out.cpu().numpy()


def oracle_extend(w, head_map=None, rows=None):
    pre, cu, kn, vn = chunk_inputs(w)
    sk, sv = oracle_prefix_stores(w)
    return oatt.extend(sk, sv, w.block_table, pre, w.q, kn, vn, cu, w.page_size, w.sm_scale, head_map=head_map,
                       quat=w.quat, rows=rows)


def check(w, head_map=None):
    print(f"extend case {w.name} {w.fmt_k}: prefix {w.prefix_lens().tolist()} new {w.new_lens().tolist()} "
          f"Hq {w.n_q_heads} Hkv {w.n_kv_heads}", flush=True)
    cache, got = run_extend(w, head_map=head_map)
    ref = oracle_extend(w, head_map=head_map)
    assert_attention_close(got, ref)
    sk, sv = oracle_stores(w)                   # every token packed: prefix + chunk
    assert_slabs_equal(cache, sk, sv)


def test_extend_iso3_scaled():
    """The ISO3 extend shape (32 query / 8 KV heads, head_dim 128) at a prefix and chunk the oracle finishes."""
    check(synth.ragged_extend([300], [200], seed=5, n_q_heads=32, n_kv_heads=8))


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
def test_extend_ragged_batch(fmt):
    """Empty, 1-cell, ragged and tile-boundary prefixes; chunks of 1, 63, 64, 65, 130 tokens."""
    check(synth.ragged_extend([0, 1, 17, 64, 200], [1, 63, 64, 65, 130], seed=22, fmt=fmt))


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
def test_extend_sequence_without_new_tokens(fmt):
    check(synth.ragged_extend([10, 40, 0], [0, 33, 5], seed=23, fmt=fmt))


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
def test_extend_uneven_head_map(fmt):
    w = synth.ragged_extend([70, 5], [40, 21], seed=24, n_q_heads=6, n_kv_heads=2, fmt=fmt)
    check(w, head_map=[1, 0, 1, 1, 0, 1])


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 1), (32, 1)])
def test_extend_group_widths(hq, hkv, fmt):
    """MHA (32 tokens per wave), MQA 16:1 and 32:1 (one token per wave)."""
    check(synth.ragged_extend([100, 37], [150, 20], seed=25 + hq, n_q_heads=hq, n_kv_heads=hkv, fmt=fmt))


def test_extend_int8_groups_of_different_scale():
    """int8 prefix whose two 64-value groups differ in scale by up to 2^12 per key (K and V), short
    and long prefixes: each group's partial sums take their own scale.  Compared relative to the
    output's magnitude (max-abs 1e-3 at unit scale)."""
    from oracle.numerics import bf16_to_f32
    w = synth.ragged_extend([1, 5, 17, 300], [3, 40, 64, 20], seed=28, fmt="int8")
    rng = np.random.default_rng(29)
    for b in range(w.batch):
        L = len(w.k[b])
        for x in (w.k, w.v):
            f = bf16_to_f32(x[b]).copy()
            f[:, :, 64:] *= (2.0 ** rng.integers(-6, 7, size=(L, w.n_kv_heads, 1))).astype(np.float32)
            x[b] = synth.bf16_bits(f)
    cache, got = run_extend(w)
    ref = oracle_extend(w)
    scale = float(np.max(np.abs(ref)))          # outputs up to 2^6 x unit scale: the bound is relative
    assert_attention_close(got / scale, ref / scale)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


def test_extend_without_packing_leaves_prefix_only():
    w = synth.ragged_extend([50], [30], seed=26)
    cache, got = run_extend(w, pack_after=False)
    assert_attention_close(got, oracle_extend(w))
    sk, sv = oracle_prefix_stores(w)
    assert_slabs_equal(cache, sk, sv)


def test_extend_deterministic():
    w = synth.ragged_extend([130], [70], seed=27)
    _, a = run_extend(w)
    _, b = run_extend(w)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
def test_extend_full_size_sampled(fmt):
    """30,000-cell ISO3 (int8) prefix + 2,048 new tokens, 32 / 8 heads, in the benchmark's launch
    configuration: every output element of every 64th query token and of the tile edges, middle and
    last tokens against the oracle; then the slabs after the deferred packing (FreeToken PR #398,
    What: the chunk's tokens are packed after its attention) byte for byte against the oracle's
    encoding of all 32,048 tokens."""
    w = synth.iso3_extend(fmt=fmt)
    rows = np.unique(np.concatenate([np.arange(0, 2048, 64), [1, 31, 32, 63, 127, 128, 1000, 1500, 2046, 2047]]))
    print(f"[extend full size] {fmt}: {len(rows)} sampled query tokens", flush=True)
    cache, got = run_extend(w)
    ref = oracle_extend(w, rows=rows)
    m = assert_attention_close(got[rows], ref[rows])
    assert np.isfinite(got).all()
    sk, sv = oracle_stores(w)                   # every token packed: prefix + chunk
    assert_slabs_equal(cache, sk, sv)
    print(f"[extend full size] {fmt}: max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}; "
          f"slabs equal after packing")
