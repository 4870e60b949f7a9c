"""Helpers shared by the tests: move seeded synthetic inputs to the device, run the library's
entry points, run the oracle on the same inputs, and compare.

Only the seeded generators in synth.py feed both sides; nothing computed by the HIP path is
ever used as an oracle input or expected value.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as oatt
from oracle import paged as opaged
from synth import Workload, dev_bf16, dev_i32, token_lists  # noqa: F401  (re-exported for the tests)

ATOL = 1e-3          # max-abs error bound on attention outputs
MIN_COS = 0.9999     # cosine bound, whole tensor and every row


def gpu_cache(w: Workload):
    import quantized_paged_kv_kvq_amd as kvq
    cache = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
    pages = kvq.Pages(dev_i32(w.block_table), dev_i32(w.seq_lens))
    return cache, pages


def gpu_append(w: Workload, cache, pages, which: str):
    import quantized_paged_kv_kvq_amd as kvq
    t = token_lists(w, which)
    if t is None:
        return
    seq, pos, k, v = t
    kvq.kvq_append(cache, pages, dev_bf16(k), dev_bf16(v), dev_i32(seq), dev_i32(pos))


def oracle_stores(w: Workload):
    """Oracle slabs holding every cell of every sequence (prefix and step tokens)."""
    sk = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = opaged.Store.empty(w.fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        opaged.append(sk, w.block_table, np.full(L, b), pos, w.k[b], w.page_size, quat=w.quat)
        opaged.append(sv, w.block_table, np.full(L, b), pos, w.v[b], w.page_size, quat=w.quat)
    return sk, sv


def tile_index(layout: str, cb: int) -> np.ndarray:
    """idx[t][c] = offset inside a (page, KV head) tile of code byte c of the cell in slot t, for the
    byte orders documented in include/kvq.h."""
    t = np.arange(16)[:, None]
    c = np.arange(cb)[None, :]
    if layout == "token":
        return t * cb + c
    if layout == "k_chunk":
        return ((c >> 4) * 16 + t) * 16 + (c & 15)
    if layout == "v_quad":
        return ((((c >> 6) << 4) | (c & 15)) * 4 + (t >> 2)) * 16 + ((c >> 4) & 3) * 4 + (t & 3)
    if layout == "v_f32":
        return ((c >> 2) * 16 + t) * 4 + (c & 3)
    if layout == "k_q4":
        return (((c >> 6) * 4 + ((c >> 2) & 3)) * 16 + t) * 16 + ((c >> 4) & 3) * 4 + (c & 3)
    raise ValueError(layout)


def store_layout(fmt: str, which: str) -> str:
    if fmt in ("iso3", "iso4"):
        return "token"
    if fmt == "q4h" and which == "k":
        return "k_q4"
    if fmt == "f32" and which == "v":
        return "v_f32"
    return "k_chunk" if which == "k" else "v_quad"


def gpu_slabs_token_major(cache, which: str):
    """The device slabs of one store as numpy, codes re-ordered to [page][head][slot][code byte]."""
    codes = (cache.k_codes if which == "k" else cache.v_codes).cpu().numpy()
    scales = (cache.k_scales if which == "k" else cache.v_scales).cpu().numpy()
    fmt = cache.fmt_k if which == "k" else cache.fmt_v
    npg, hkv, nbytes = codes.shape
    cb = nbytes // 16
    idx = tile_index(store_layout(fmt, which), cb)
    assert sorted(idx.ravel().tolist()) == list(range(nbytes)), "tile byte order must be a permutation"
    return np.ascontiguousarray(codes[:, :, idx]), scales


def assert_slabs_equal(cache, sk, sv):
    for which, st in (("k", sk), ("v", sv)):
        codes, scales = gpu_slabs_token_major(cache, which)
        bad = np.argwhere(codes != st.codes)
        assert len(bad) == 0, f"{which} codes differ at {len(bad)} bytes, first {bad[:5].tolist()}"
        sb = scales.view(np.uint16)
        ob = st.scales.view(np.uint16)
        bad = np.argwhere(sb != ob)
        assert len(bad) == 0, (f"{which} scales differ at {len(bad)} places, first {bad[:5].tolist()} "
                               f"gpu={sb[tuple(bad[0])]:#06x} oracle={ob[tuple(bad[0])]:#06x}")


def oracle_decode(w: Workload, sk, sv, head_map=None, seqs=None):
    return oatt.decode(sk, sv, w.block_table, w.seq_lens, w.q, w.page_size, w.sm_scale, q_lens=w.q_lens,
                       head_map=head_map, quat=w.quat, seqs=seqs)


def attention_errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, whole-tensor cosine, min row cosine over rows that are not all zero)."""
    g = got.astype(np.float64).reshape(-1, got.shape[-1])
    r = ref.astype(np.float64).reshape(-1, ref.shape[-1])
    maxabs = float(np.max(np.abs(g - r))) if g.size else 0.0
    cos = float(np.sum(g * r) / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300)) if g.size else 1.0
    rn, gn = np.linalg.norm(r, axis=1), np.linalg.norm(g, axis=1)
    live = rn > 0
    row_cos = np.sum(g[live] * r[live], axis=1) / np.maximum(gn[live] * rn[live], 1e-300)
    assert np.all(gn[~live] == 0), "rows with no visible cell must be exactly zero"
    return maxabs, cos, float(row_cos.min()) if live.any() else 1.0


def assert_attention_close(got, ref, atol=ATOL, min_cos=MIN_COS):
    maxabs, cos, row_cos = attention_errors(got, ref)
    assert maxabs <= atol and cos > min_cos and row_cos > min_cos, \
        f"max-abs {maxabs:.3e} (<= {atol}), cosine {cos:.7f}, min row cosine {row_cos:.7f} (> {min_cos})"
    return maxabs, cos, row_cos
