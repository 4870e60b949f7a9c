"""Guard bands around the cache slabs (GPU): every kernel that writes cells -- append, the fused
decode step's quantize-on-write, extend's packing -- stays inside the slabs it is given.

Each of the four slabs (K and V codes, K and V scales or norms) is a view into an allocation with
guard pages before and after it, every guard byte set to a sentinel.  After the writes (and the reads
of decode, verify and gather over the same slabs) every guard byte must still hold the sentinel, and
the slabs themselves must equal the oracle's encoding byte for byte.  The page tables are seeded
permutations of the whole pool, so the first and the last page of every slab are written.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import assert_slabs_equal, dev_bf16, dev_i32, gpu_append, gpu_cache, oracle_stores
from test_gpu_extend import chunk_inputs

pytestmark = pytest.mark.gpu

GUARD = 2                  # guard pages before and after each slab
SENTINEL = 0xA5


def guard(cache):
    """Move the cache's slabs into guarded allocations; returns [(name, whole allocation)]."""
    import torch
    out = []
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        t = getattr(cache, name)
        whole = torch.empty((t.shape[0] + 2 * GUARD,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        whole.view(torch.uint8).fill_(SENTINEL)
        inner = whole[GUARD:GUARD + t.shape[0]]
        inner.zero_()
        setattr(cache, name, inner)
        out.append((name, whole))
    cache._desc = None                       # the descriptor takes the new slab addresses
    return out


def assert_guards(guards):
    import torch
    torch.cuda.synchronize()
    for name, whole in guards:
        b = whole.view(torch.uint8)
        for side, part in (("before", b[:GUARD]), ("after", b[-GUARD:])):
            bad = int((part != SENTINEL).sum())
            assert bad == 0, f"{name}: {bad} guard bytes {side} the slab changed"


MIXES = [("int8", "int8", 128), ("int8", "int8", 64), ("int8", "q4h", 256), ("q4h", "q4h", 256),
         ("iso3", "iso3", 128), ("iso3", "iso3", 256), ("iso4", "iso4", 256), ("int8", "f32", 256),
         ("f32", "int8", 128)]


@pytest.mark.parametrize("fk,fv,D", MIXES, ids=[f"{a}-{b}-{d}" for a, b, d in MIXES])
def test_append_decode_gather_stay_inside(fk, fv, D):
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_decode(fk, fv, [37, 64, 5, 1, 130, 16], seed=31, n_q_heads=8, n_kv_heads=2, head_dim=D)
    print(f"[guard] append + decode + gather {fk}/{fv} D={D}", flush=True)
    cache, pages = gpu_cache(w)
    guards = guard(cache)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    kvq.kvq_decode_attn(cache, pages, dev_bf16(w.q), sm_scale=w.sm_scale)
    for which in ("k", "v"):
        for b in range(w.batch):
            L = int(w.seq_lens[b])
            if L:
                kvq.kvq_dequant_gather(cache, pages, which, b, 0, L)
    assert_guards(guards)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


BULK = [("int8", "int8", 128), ("int8", "q4h", 256), ("q4h", "q4h", 256), ("int8", "f32", 256), ("f32", "int8", 256),
        ("iso3", "iso3", 128), ("iso3", "iso3", 256), ("iso4", "iso4", 256)]


@pytest.mark.parametrize("fk,fv,D", BULK, ids=[f"{a}-{b}-{d}" for a, b, d in BULK])
def test_bulk_append_stays_inside(fk, fv, D):
    """A multi-token append large enough that the int8 and q4_0 encoders take 4 cells per thread and
    the ISO encoders 4 blocks per wave (more than two rounds of the CUs at one per thread), with
    ragged sequence ends; in the mixed cases the two stores' grids differ in size."""
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_decode(fk, fv, [8191, 3, 4100], seed=34, n_q_heads=8, n_kv_heads=2, head_dim=D)
    print(f"[guard] bulk append {fk}/{fv} D={D}", flush=True)
    cache, pages = gpu_cache(w)
    guards = guard(cache)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    assert_guards(guards)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


FUSED = [("int8", "int8", 128, 1), ("int8", "q4h", 256, 1), ("int8", "q4h", 256, 3), ("int8", "f32", 256, 1),
         ("f32", "int8", 128, 1)]


@pytest.mark.parametrize("fk,fv,D,n_q", FUSED, ids=[f"{a}-{b}-{d}-q{n}" for a, b, d, n in FUSED])
def test_fused_step_stays_inside(fk, fv, D, n_q):
    """The fused decode step writes the step's cells (the last n_q of each sequence) from inside the
    attention launch."""
    import quantized_paged_kv_kvq_amd as kvq
    back = list(range(n_q - 1, -1, -1)) if n_q > 1 else None
    hq = 8 if n_q * 4 <= 32 else 4
    w = synth.ragged_decode(fk, fv, [37, 64, n_q + 3, 130, 16], seed=32, n_q=n_q, q_len_back=back, n_q_heads=hq,
                            n_kv_heads=2, head_dim=D)
    print(f"[guard] fused step {fk}/{fv} D={D} n_q={n_q}", flush=True)
    cache, pages = gpu_cache(w)
    guards = guard(cache)
    gpu_append(w, cache, pages, "prefix")
    ks = np.stack([w.k[b][int(w.seq_lens[b]) - n_q:int(w.seq_lens[b])] for b in range(w.batch)])
    vs = np.stack([w.v[b][int(w.seq_lens[b]) - n_q:int(w.seq_lens[b])] for b in range(w.batch)])
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    kvq.kvq_decode_attn_append(cache, pages, dev_bf16(ks), dev_bf16(vs), dev_bf16(w.q), q_lens=q_lens,
                               sm_scale=w.sm_scale)
    assert_guards(guards)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)


@pytest.mark.parametrize("fmt", ["iso3", "int8"])
def test_extend_packing_stays_inside(fmt):
    """Extend over a packed prefix, then the chunk's tokens packed into their cells."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_extend([0, 17, 64, 200], [63, 64, 65, 130], seed=33, fmt=fmt)
    print(f"[guard] extend + pack {fmt}", flush=True)
    pre, cu, kn, vn = chunk_inputs(w)
    cache = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
    guards = guard(cache)
    pages = kvq.Pages(dev_i32(w.block_table), dev_i32(pre))
    tok_seq = np.concatenate([np.full(int(pre[b]), b, np.int32) for b in range(w.batch)])
    tok_pos = np.concatenate([np.arange(int(pre[b]), dtype=np.int32) for b in range(w.batch)])
    kp = np.concatenate([w.k[b][:int(pre[b])] for b in range(w.batch)])
    vp = np.concatenate([w.v[b][:int(pre[b])] for b in range(w.batch)])
    kvq.kvq_append(cache, pages, dev_bf16(kp), dev_bf16(vp), dev_i32(tok_seq), dev_i32(tok_pos))
    out = kvq.kvq_extend_attn(cache, pages, dev_bf16(w.q), dev_bf16(kn), dev_bf16(vn), dev_i32(cu),
                              int(w.new_lens().max()), sm_scale=w.sm_scale, pack_after=True)
    torch.cuda.synchronize()
    assert_guards(guards)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    assert np.isfinite(out.cpu().numpy()).all()        # (attention parity is the extend tests' job)
