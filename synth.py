"""Seeded synthetic inputs for the quantized paged KV cache.

This module is shared by the CPU oracle's tests, the GPU parity tests, ``smoke()``
and ``bench.py``.  It holds none of the method's arithmetic: it draws normal
samples, rounds them to bfloat16 bit patterns, builds page tables and lengths,
and draws the one rotation quaternion the ISO3 format uses (a random input of
the method, passed to both sides).

Workloads follow the shapes the pages measure on:
  * strata PR #2698 (int8 K/V caches), section Measurements: 64K / 128K contexts,
    head_dim 256 with 2 KV heads;
  * strata PR #120 (k8v4 hybrid), section Measured: ~118.75k-token context,
    MTP verify windows (section Tests: per-query step arrays);
  * FreeToken PR #398 (ISO3/ISO4), section Why: a 30k-token prompt prefilled
    over a packed prefix.
The models and prompts themselves are not used: every K, V and q value is a
seeded N(0, 1) sample rounded to bfloat16.

Draw order per workload: page-table permutation, K, V, q, then the quaternion.
Large multi-sequence workloads draw each sequence from its own sub-seed
``seed * 1000 + b`` so they can be generated one sequence at a time.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE_SIZE = 16


def bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, outlier_channels=None, outlier_scale=20.0) -> np.ndarray:
    """N(0, 1) float32 samples (optionally with some last-axis channels scaled) as bf16 bits."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_channels is not None and len(outlier_channels):
        x[..., np.asarray(outlier_channels)] *= np.float32(outlier_scale)
    return bf16_bits(x)


def random_quaternion(seed: int) -> np.ndarray:
    """One seeded unit quaternion (w, x, y, z): 4 fp64 normals, normalised in fp64, rounded to fp32."""
    g = np.random.default_rng(seed).standard_normal(4)
    return (g / np.sqrt(np.sum(g * g))).astype(np.float32)


@dataclass
class Workload:
    """One step of the hot path over a seeded synthetic cache.

    ``seq_lens[b]`` is the context length of sequence b after the step's append.
    ``k[b]`` / ``v[b]`` hold the bf16 bits of all ``seq_lens[b]`` tokens, shape
    ``[seq_lens[b]][n_kv_heads][head_dim]``; the last ``n_step`` of them are the
    tokens the step itself writes (quantize-on-write), the rest pre-fill the cache.
    For extend workloads ``n_step`` is the number of new (bf16) tokens, which
    the step attends unquantised and packs afterwards.
    """
    name: str
    fmt_k: str                      # 'int8' | 'q4h' | 'iso3' | 'f32'
    fmt_v: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens: np.ndarray            # int32 [B]
    block_table: np.ndarray         # int32 [B][max_pages]
    num_pages: int
    k: List[np.ndarray]             # per sequence, uint16 bf16 bits
    v: List[np.ndarray]
    q: np.ndarray                   # uint16 [B][n_q][Hq][D] (decode) or [n_new_total][Hq][D] (extend)
    n_q: int = 1
    n_step: int = 1
    q_lens: Optional[np.ndarray] = None   # int32 [B][n_q] or None (every row uses seq_lens)
    quat: np.ndarray = field(default_factory=lambda: np.array([1, 0, 0, 0], np.float32))
    kind: str = "decode"            # 'decode' | 'extend'
    sm_scale: float = 0.0
    meta: dict = field(default_factory=dict)

    def __post_init__(self):
        if not self.sm_scale:
            self.sm_scale = float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def new_lens(self) -> np.ndarray:
        """Tokens the step itself writes, per sequence."""
        if "new" in self.meta:
            return np.asarray(self.meta["new"], np.int32)
        return np.full(self.batch, self.n_step, np.int32)

    def prefix_lens(self) -> np.ndarray:
        """Cells already in the cache before the step writes."""
        return (self.seq_lens - self.new_lens()).astype(np.int32)


def _page_table(rng, lens, page_size, identity):
    """Give each sequence ceil(len/page) pages from one pool; the pool order is a seeded permutation."""
    need = [(int(L) + page_size - 1) // page_size for L in lens]
    total = int(sum(need))
    perm = np.arange(total, dtype=np.int32) if identity else rng.permutation(total).astype(np.int32)
    max_pages = max(max(need), 1)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    # Unused tail entries point at page 0 so that a table row is always a valid index list;
    # kernels never read past ceil(len/page).
    table[table < 0] = 0
    return table, max(total, 1)


def tiny_int8_decode(seed: int = 1, ctx: int = 512, n_q_heads: int = 4, n_kv_heads: int = 1,
                     head_dim: int = 128) -> Workload:
    """Batch 1, GQA 4:1, head_dim 128, context 512, identity page table."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=True)
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, 1, n_q_heads, head_dim))
    return Workload("tiny_int8_decode", "int8", "int8", 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                    lens, table, npages, [k], [v], q)


def moe_int8_decode(ctx: int = 131072, seed: int = 2, n_q_heads: int = 16, n_kv_heads: int = 2,
                    head_dim: int = 256, n_outliers: int = 4) -> Workload:
    """One full-attention layer of a Qwen3.5-MoE-style model: GQA 16:2, head_dim 256,
    random page table, K with a few seeded outlier channels scaled x20."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    outliers = np.sort(rng.choice(head_dim, size=n_outliers, replace=False)) if n_outliers else []
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim), outlier_channels=outliers)
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, 1, n_q_heads, head_dim))
    w = Workload("moe_int8_decode", "int8", "int8", 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                 lens, table, npages, [k], [v], q)
    w.meta["outlier_channels"] = [int(c) for c in outliers]
    return w


def batched_int8_decode(seed: int = 3, n_seqs: int = 32, len_lo: int = 4096, len_hi: int = 32768,
                        n_q_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128) -> Workload:
    """Many sequences of mixed length, GQA 32:8, head_dim 128; every step appends one
    token per sequence (quantize-on-write) and then decodes."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi, size=n_seqs, endpoint=True).astype(np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    q = normal_bf16(rng, (n_seqs, 1, n_q_heads, head_dim))
    ks, vs = [], []
    for b in range(n_seqs):
        sub = np.random.default_rng(seed * 1000 + b)
        ks.append(normal_bf16(sub, (int(lens[b]), n_kv_heads, head_dim)))
        vs.append(normal_bf16(sub, (int(lens[b]), n_kv_heads, head_dim)))
    return Workload("batched_int8_decode", "int8", "int8", n_seqs, n_q_heads, n_kv_heads, head_dim,
                    PAGE_SIZE, lens, table, npages, ks, vs, q)


def batched_iso3_decode(seed: int = 6, n_seqs: int = 32, len_lo: int = 4096, len_hi: int = 32768,
                        n_q_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128) -> Workload:
    """batched_int8_decode's shapes over ISO3 K and V stores (one seeded rotation quaternion)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi, size=n_seqs, endpoint=True).astype(np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    q = normal_bf16(rng, (n_seqs, 1, n_q_heads, head_dim))
    ks, vs = [], []
    for b in range(n_seqs):
        sub = np.random.default_rng(seed * 1000 + b)
        ks.append(normal_bf16(sub, (int(lens[b]), n_kv_heads, head_dim)))
        vs.append(normal_bf16(sub, (int(lens[b]), n_kv_heads, head_dim)))
    quat = random_quaternion(seed + 1000)
    return Workload("batched_iso3_decode", "iso3", "iso3", n_seqs, n_q_heads, n_kv_heads, head_dim,
                    PAGE_SIZE, lens, table, npages, ks, vs, q, quat=quat)


def moe_iso3_decode(ctx: int = 131072, seed: int = 7, n_q_heads: int = 16, n_kv_heads: int = 2,
                    head_dim: int = 256, n_outliers: int = 4, fmt: str = "iso3") -> Workload:
    """moe_int8_decode's layer (GQA 16:2, head_dim 256, K outlier channels x20) over ISO3 (or, with
    fmt="iso4", ISO4) K and V."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    outliers = np.sort(rng.choice(head_dim, size=n_outliers, replace=False)) if n_outliers else []
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim), outlier_channels=outliers)
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, 1, n_q_heads, head_dim))
    quat = random_quaternion(seed + 1000)
    w = Workload(f"moe_{fmt}_decode", fmt, fmt, 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                 lens, table, npages, [k], [v], q, quat=quat)
    w.meta["outlier_channels"] = [int(c) for c in outliers]
    return w


def moe_q4h_decode(ctx: int = 131072, seed: int = 8, n_q_heads: int = 16, n_kv_heads: int = 2,
                   head_dim: int = 256, n_outliers: int = 4) -> Workload:
    """moe_int8_decode's layer (GQA 16:2, head_dim 256, K outlier channels x20) over Hadamard-rotated
    q4_0 K and V stores (strata PR #2698, "Not in this PR": rotate K and V, the queries and the output)."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    outliers = np.sort(rng.choice(head_dim, size=n_outliers, replace=False)) if n_outliers else []
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim), outlier_channels=outliers)
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, 1, n_q_heads, head_dim))
    w = Workload("moe_q4h_decode", "q4h", "q4h", 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                 lens, table, npages, [k], [v], q)
    w.meta["outlier_channels"] = [int(c) for c in outliers]
    return w


def moe_single_store_decode(fmt_k: str = "int8", fmt_v: str = "f32", ctx: int = 131072, seed: int = 9,
                            n_q: int = 1, n_q_heads: int = 16, n_kv_heads: int = 2, head_dim: int = 256,
                            n_outliers: int = 4) -> Workload:
    """moe_int8_decode's layer (GQA 16:2, head_dim 256, K outlier channels x20) with one store
    quantised and the other FP32 (strata PR #2698: `k8v32` / `k32v8`, measured there at 64K on a
    Qwen3.6-35B-A3B model with a 2-token MTP draft); n_q > 1 makes a verify window of causal lengths
    ctx - n_q + 1 .. ctx."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    outliers = np.sort(rng.choice(head_dim, size=n_outliers, replace=False)) if n_outliers else []
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim), outlier_channels=outliers)
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, n_q, n_q_heads, head_dim))
    name = {("int8", "f32"): "moe_k8v32_decode", ("f32", "int8"): "moe_k32v8_decode"}.get((fmt_k, fmt_v),
                                                                                          "moe_f32_decode")
    w = Workload(name, fmt_k, fmt_v, 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE, lens, table, npages, [k], [v],
                 q, n_q=n_q, n_step=n_q)
    if n_q > 1:
        w.q_lens = (ctx - n_q + 1 + np.arange(n_q, dtype=np.int32))[None, :]
    w.meta["outlier_channels"] = [int(c) for c in outliers]
    return w


def k8v4_verify(ctx: int = 118750, seed: int = 4, n_q: int = 3, n_q_heads: int = 16,
                n_kv_heads: int = 2, head_dim: int = 256) -> Workload:
    """int8 K + Hadamard-rotated q4_0 V; an MTP verify window of ``n_q`` query tokens whose
    causal lengths are ctx-n_q+1 ... ctx (the window's own tokens are the step's appends)."""
    rng = np.random.default_rng(seed)
    lens = np.array([ctx], np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    k = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    v = normal_bf16(rng, (ctx, n_kv_heads, head_dim))
    q = normal_bf16(rng, (1, n_q, n_q_heads, head_dim))
    q_lens = (ctx - n_q + 1 + np.arange(n_q, dtype=np.int32))[None, :].astype(np.int32)
    return Workload("k8v4_verify", "int8", "q4h", 1, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                    lens, table, npages, [k], [v], q, n_q=n_q, n_step=n_q, q_lens=q_lens)


def iso3_extend(prefix: int = 30000, n_new: int = 2048, seed: int = 5, n_q_heads: int = 32,
                n_kv_heads: int = 8, head_dim: int = 128, batch: int = 1, fmt: str = "iso3") -> Workload:
    """Prefill chunk over an ISO3-packed (fmt="int8": int8-g64) prefix: ``n_new`` bf16 tokens per
    sequence attend the packed prefix plus themselves causally, and are packed after the attention."""
    rng = np.random.default_rng(seed)
    lens = np.full(batch, prefix + n_new, np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=False)
    ks = [normal_bf16(rng, (prefix + n_new, n_kv_heads, head_dim)) for _ in range(batch)]
    vs = [normal_bf16(rng, (prefix + n_new, n_kv_heads, head_dim)) for _ in range(batch)]
    q = normal_bf16(rng, (batch * n_new, n_q_heads, head_dim))
    quat = random_quaternion(seed + 1000)
    return Workload(f"{fmt}_extend", fmt, fmt, batch, n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                    lens, table, npages, ks, vs, q, n_q=n_new, n_step=n_new, quat=quat, kind="extend")


def ragged_decode(fmt_k: str, fmt_v: str, lens, seed: int = 11, n_q: int = 1, n_q_heads: int = 8,
                  n_kv_heads: int = 2, head_dim: int = 128, identity: bool = False,
                  q_len_back: Optional[List[int]] = None) -> Workload:
    """Small decode/verify cases of any format mix with ragged lengths, for parity tests.
    ``q_len_back[t]`` makes query t attend ``seq_lens[b] - q_len_back[t]`` cells."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=identity)
    ks = [normal_bf16(rng, (int(L), n_kv_heads, head_dim)) for L in lens]
    vs = [normal_bf16(rng, (int(L), n_kv_heads, head_dim)) for L in lens]
    q = normal_bf16(rng, (len(lens), n_q, n_q_heads, head_dim))
    q_lens = None
    if q_len_back is not None:
        q_lens = np.maximum(lens[:, None] - np.asarray(q_len_back, np.int32)[None, :], 0).astype(np.int32)
    quat = random_quaternion(seed + 1000)
    n_step = min(n_q, int(lens.min())) if len(lens) else 0
    return Workload("ragged_decode", fmt_k, fmt_v, len(lens), n_q_heads, n_kv_heads, head_dim,
                    PAGE_SIZE, lens, table, npages, ks, vs, q, n_q=n_q, n_step=n_step, q_lens=q_lens,
                    quat=quat)


def ragged_extend(prefix_lens, new_lens, seed: int = 21, n_q_heads: int = 8, n_kv_heads: int = 2,
                  head_dim: int = 128, identity: bool = False, fmt: str = "iso3") -> Workload:
    """Prefill chunks over ISO3 prefixes of any lengths, for parity tests: sequence b holds
    ``prefix_lens[b]`` packed cells and ``new_lens[b]`` new bf16 tokens; the q rows of all
    sequences' new tokens are concatenated in sequence order."""
    rng = np.random.default_rng(seed)
    pre = np.asarray(prefix_lens, np.int32)
    new = np.asarray(new_lens, np.int32)
    lens = (pre + new).astype(np.int32)
    table, npages = _page_table(rng, lens, PAGE_SIZE, identity=identity)
    ks = [normal_bf16(rng, (int(L), n_kv_heads, head_dim)) for L in lens]
    vs = [normal_bf16(rng, (int(L), n_kv_heads, head_dim)) for L in lens]
    q = normal_bf16(rng, (int(new.sum()), n_q_heads, head_dim))
    quat = random_quaternion(seed + 1000)
    return Workload("ragged_extend", fmt, fmt, len(lens), n_q_heads, n_kv_heads, head_dim, PAGE_SIZE,
                    lens, table, npages, ks, vs, q, n_q=int(new.max()) if len(new) else 0, n_step=0, quat=quat,
                    kind="extend", meta={"new": new})


# ---------------------------------------------------------------------------------------------
# Moving a workload to the device (torch is imported only when these are called)

def dev_bf16(bits):
    """uint16 bf16 bit patterns -> a torch.bfloat16 tensor on the current GPU."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_i32(a):
    """An integer array -> a torch.int32 tensor on the current GPU."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def token_lists(w: "Workload", which: str):
    """(tok_seq, tok_pos, K rows, V rows) of the tokens that pre-fill the cache ('prefix') or of the
    step's own tokens ('step'), ordered by sequence, then position; None when there are none."""
    seqs, poss, rows = [], [], []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        P = L - w.n_step
        lo, hi = (0, P) if which == "prefix" else (max(P, 0), L)
        if hi <= lo:
            continue
        seqs.append(np.full(hi - lo, b, np.int32))
        poss.append(np.arange(lo, hi, dtype=np.int32))
        rows.append((w.k[b][lo:hi], w.v[b][lo:hi]))
    if not seqs:
        return None
    return (np.concatenate(seqs), np.concatenate(poss), np.concatenate([r[0] for r in rows]),
            np.concatenate([r[1] for r in rows]))
