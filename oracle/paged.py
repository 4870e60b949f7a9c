"""Paged slabs of quantised cells and their addressing (oracle; test infrastructure only).

The cache is paged (FreeToken PR #398, section "What": a paged KV pool; strata
PR #120, section "Tests": append/gather through a non-identity page table).
Codes and scales live in separate arrays (strata PR #2698, section "What it
does": int8 codes and their FP16 scales are separate buffers).  An unquantised
FP32 store keeps its binary32 values in the code bytes and has no scales.

Layout of one store (K or V) -- the same layout the library documents:
    codes  uint8   [num_pages][n_kv_heads][page_size][code_bytes]
    scales float16 [num_pages][n_kv_heads][page_size][n_scales]
Logical token j of sequence b lives in page ``block_table[b][j // page_size]``
at slot ``j % page_size``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import f32, int8_g64, iso3, iso4, q4h
from .numerics import bf16_to_f32

FORMATS = {"int8": int8_g64, "q4h": q4h, "iso3": iso3, "iso4": iso4, "f32": f32}


def cell_bytes(fmt: str, head_dim: int):
    """(code bytes, fp16 scale count) per (token, KV head) cell of one store."""
    m = FORMATS[fmt]
    return m.code_bytes(head_dim), m.n_scales(head_dim)


@dataclass
class Store:
    fmt: str
    codes: np.ndarray      # uint8 [num_pages][Hkv][P][code_bytes]
    scales: np.ndarray     # float16 [num_pages][Hkv][P][n_scales]

    @staticmethod
    def empty(fmt, num_pages, n_kv_heads, page_size, head_dim):
        cb, ns = cell_bytes(fmt, head_dim)
        return Store(fmt, np.zeros((num_pages, n_kv_heads, page_size, cb), np.uint8),
                     np.zeros((num_pages, n_kv_heads, page_size, ns), np.float16))


def locate(block_table: np.ndarray, seq: np.ndarray, pos: np.ndarray, page_size: int):
    """(page, slot) of logical positions ``pos`` of sequences ``seq``."""
    seq = np.asarray(seq, np.int64)
    pos = np.asarray(pos, np.int64)
    return block_table[seq, pos // page_size].astype(np.int64), pos % page_size


def encode_cells(fmt: str, x_f32: np.ndarray, quat=None):
    """Encode float32 head vectors [..., D] into (code bytes [..., cb], scales [..., ns])."""
    if fmt == "int8":
        codes, scales = int8_g64.encode(x_f32)
        return codes.view(np.uint8), scales
    if fmt == "q4h":
        return q4h.encode(x_f32)
    if fmt == "iso3":
        return iso3.encode(x_f32, quat)
    if fmt == "iso4":
        return iso4.encode(x_f32, quat)
    if fmt == "f32":
        return f32.encode(x_f32)
    raise ValueError(fmt)


def decode_cells(fmt: str, codes: np.ndarray, scales: np.ndarray, quat=None, rotated: bool = True):
    """Dequantise cells.  For q4h, ``rotated`` keeps the stored (Hadamard) basis in binary32;
    otherwise the values are rotated back in fp64."""
    if fmt == "int8":
        return int8_g64.decode(codes.view(np.int8), scales)
    if fmt == "q4h":
        return q4h.decode_rotated(codes, scales) if rotated else q4h.decode(codes, scales)
    if fmt == "iso3":
        return iso3.decode(codes, scales, quat)
    if fmt == "iso4":
        return iso4.decode(codes, scales, quat)
    if fmt == "f32":
        return f32.decode(codes, scales)
    raise ValueError(fmt)


def append(store: Store, block_table, tok_seq, tok_pos, x_bf16, page_size, quat=None, chunk=65536):
    """Quantise-on-write: encode the bf16 vectors x[i] ([n_tok][Hkv][D]) into the cells of
    (tok_seq[i], tok_pos[i]).  Tokens are encoded independently, so chunking changes nothing."""
    tok_seq = np.asarray(tok_seq)
    tok_pos = np.asarray(tok_pos)
    for s in range(0, len(tok_seq), chunk):
        e = min(s + chunk, len(tok_seq))
        codes, scales = encode_cells(store.fmt, bf16_to_f32(x_bf16[s:e]), quat)
        page, slot = locate(block_table, tok_seq[s:e], tok_pos[s:e], page_size)
        store.codes[page, :, slot, :] = codes
        store.scales[page, :, slot, :] = scales


def gather_raw(store: Store, block_table, seq: int, start: int, count: int, page_size: int):
    """Code bytes and scales of cells [start, start+count) of one sequence: ([count][Hkv][cb], [count][Hkv][ns])."""
    pos = np.arange(start, start + count)
    page, slot = locate(block_table, np.full(count, seq), pos, page_size)
    return store.codes[page, :, slot, :], store.scales[page, :, slot, :]


def gather(store: Store, block_table, seq: int, start: int, count: int, page_size: int, quat=None,
           rotated: bool = True) -> np.ndarray:
    """Dequantised values of cells [start, start+count) of one sequence: [count][Hkv][D]."""
    codes, scales = gather_raw(store, block_table, seq, start, count, page_size)
    return decode_cells(store.fmt, codes, scales, quat, rotated)
