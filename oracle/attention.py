"""Softmax attention over dequantised K/V, in fp64 (oracle; test infrastructure only).

What the kernels compute is plain scaled-dot-product attention over the values
the cache holds: the split-K partials, online softmax, log-sum-exp combine,
rotated-basis accumulation and MFMA tiling are only faster routes to it.  So
this module writes the definition out:

    s_j = sm_scale * <q, K_j>,  w_j = exp(s_j - max s),  o = sum_j w_j V_j / sum_j w_j

with K_j, V_j the dequantised cells (binary32 widened to fp64; the q4h V side is
rotated back by H in fp64).  A query with no visible keys returns zeros.

Paths (FreeToken PR #398, section "What"; strata PR #2698, section "What it
does"; strata PR #120, sections "How" and "Tests"):
  * decode   -- one query token per sequence over its cached cells;
  * verify   -- several query tokens per sequence, each with its own causal
    length (the per-query step arrays of an MTP verify window);
  * extend   -- a prefill chunk: query i of a sequence with P cached cells attends
    the P dequantised cells plus new tokens 0..i *unquantised* (bf16), because
    the chunk's own tokens are packed only after its attention.
GQA: query head h reads KV head ``head_map[h]`` (default h // (Hq / Hkv)).
"""
from __future__ import annotations

import numpy as np

from . import paged
from .numerics import bf16_to_f32


def default_head_map(n_q_heads: int, n_kv_heads: int) -> np.ndarray:
    return (np.arange(n_q_heads) // (n_q_heads // n_kv_heads)).astype(np.int32)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [R][D], K [L][D], V [L][D] (fp64) -> fp64 [R][D]; every row sees all L keys."""
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]), np.float64)
    s = float(sm_scale) * (q @ K.T)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=1, keepdims=True)


def attend_lengths(q: np.ndarray, K: np.ndarray, V: np.ndarray, lengths, sm_scale: float,
                   chunk: int = 256) -> np.ndarray:
    """Row r sees keys [0, lengths[r]); keys past a row's length get weight exactly 0."""
    lengths = np.asarray(lengths, np.int64)
    out = np.zeros((q.shape[0], V.shape[1]), np.float64)
    for s in range(0, q.shape[0], chunk):
        L = lengths[s:s + chunk]
        Lmax = int(L.max()) if len(L) else 0
        if Lmax == 0:
            continue
        sc = float(sm_scale) * (q[s:s + chunk] @ K[:Lmax].T)
        visible = np.arange(Lmax)[None, :] < L[:, None]
        sc = np.where(visible, sc, -np.inf)
        m = sc.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        w = np.exp(sc - m)
        den = w.sum(axis=1, keepdims=True)
        out[s:s + chunk] = (w @ V[:Lmax]) / np.where(den > 0, den, 1.0)
    return out


def _dequant_seq(store, block_table, b, count, page_size, quat):
    x = paged.gather(store, block_table, b, 0, count, page_size, quat=quat, rotated=False)
    return np.asarray(x, dtype=np.float64)


def decode(store_k, store_v, block_table, seq_lens, q_bf16, page_size, sm_scale,
           q_lens=None, head_map=None, quat=None, seqs=None) -> np.ndarray:
    """Decode / verify attention.  q_bf16: uint16 [B][n_q][Hq][D]; q_lens: [B][n_q] or None.
    Returns float32 [B][n_q][Hq][D] (rows of sequences not in ``seqs`` stay zero)."""
    q_bf16 = np.asarray(q_bf16)
    B, n_q, Hq, D = q_bf16.shape
    Hkv = store_k.codes.shape[1]
    hmap = default_head_map(Hq, Hkv) if head_map is None else np.asarray(head_map)
    out = np.zeros((B, n_q, Hq, D), np.float32)
    q = bf16_to_f32(q_bf16).astype(np.float64)
    for b in (range(B) if seqs is None else seqs):
        lens = np.full(n_q, int(seq_lens[b])) if q_lens is None else np.asarray(q_lens[b])
        Lmax = int(lens.max()) if n_q else 0
        K = _dequant_seq(store_k, block_table, b, Lmax, page_size, quat)
        V = _dequant_seq(store_v, block_table, b, Lmax, page_size, quat)
        for kh in range(Hkv):
            heads = np.nonzero(hmap == kh)[0]
            if len(heads) == 0:
                continue
            rows = q[b][:, heads, :].reshape(-1, D)                 # (t, h) rows of this KV head
            row_lens = np.repeat(lens, len(heads))
            o = attend_lengths(rows, K[:, kh, :], V[:, kh, :], row_lens, sm_scale)
            out[b][:, heads, :] = o.reshape(n_q, len(heads), D).astype(np.float32)
    return out


def extend(store_k, store_v, block_table, prefix_lens, q_bf16, k_new_bf16, v_new_bf16, cu_new,
           page_size, sm_scale, head_map=None, quat=None, rows=None) -> np.ndarray:
    """Prefill-chunk attention.  q_bf16: [N][Hq][D]; k/v_new_bf16: [N][Hkv][D]; cu_new: [B+1].
    New token i of sequence b sits at position prefix_lens[b] + i and attends the dequantised
    prefix plus new tokens 0..i as bf16.  ``rows`` limits the work to some global query rows.
    Returns float32 [N][Hq][D]."""
    q_bf16 = np.asarray(q_bf16)
    N, Hq, D = q_bf16.shape
    Hkv = store_k.codes.shape[1]
    hmap = default_head_map(Hq, Hkv) if head_map is None else np.asarray(head_map)
    out = np.zeros((N, Hq, D), np.float32)
    want = np.ones(N, bool) if rows is None else np.isin(np.arange(N), rows)
    for b in range(len(cu_new) - 1):
        s, e = int(cu_new[b]), int(cu_new[b + 1])
        sel = np.nonzero(want[s:e])[0]
        if len(sel) == 0:
            continue
        P = int(prefix_lens[b])
        Kp = _dequant_seq(store_k, block_table, b, P, page_size, quat)
        Vp = _dequant_seq(store_v, block_table, b, P, page_size, quat)
        Kn = bf16_to_f32(k_new_bf16[s:e]).astype(np.float64)
        Vn = bf16_to_f32(v_new_bf16[s:e]).astype(np.float64)
        K = np.concatenate([Kp, Kn], axis=0)
        V = np.concatenate([Vp, Vn], axis=0)
        q = bf16_to_f32(q_bf16[s:e]).astype(np.float64)
        lens = P + sel + 1
        for kh in range(Hkv):
            heads = np.nonzero(hmap == kh)[0]
            if len(heads) == 0:
                continue
            rows = q[sel][:, heads, :].reshape(-1, D)
            row_lens = np.repeat(lens, len(heads))
            o = attend_lengths(rows, K[:, kh, :], V[:, kh, :], row_lens, sm_scale)
            out[s + sel[:, None], heads[None, :], :] = o.reshape(len(sel), len(heads), D).astype(np.float32)
    return out
