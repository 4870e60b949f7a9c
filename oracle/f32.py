"""Unquantised binary32 cache cells (oracle; test infrastructure only).

strata PR #2698 (intro and section "What it does"): the engine's caches are FP32 by default, 2 KiB
per cell per store at head_dim 256 over its two KV heads, and the modes `k8v32` / `k32v8` quantise
only one of the two stores (int8 codes + FP16 scales) and keep the other in FP32.

Readings where the pages are silent:
  * a cell of the FP32 store holds the D binary32 values of its head vector, little-endian, value d
    in code bytes 4d .. 4d+3, with no scales;
  * values written from bf16 inputs are the bf16 values exactly (a bf16 number is the upper half of
    the binary32 number with the same value), so writing and reading back changes nothing.
"""
from __future__ import annotations

import numpy as np


def code_bytes(head_dim: int) -> int:
    return 4 * head_dim


def n_scales(head_dim: int) -> int:
    return 0


def encode(x: np.ndarray):
    """x: float32 [..., D] -> (bytes uint8 [..., 4D], scales float16 [..., 0])."""
    x = np.ascontiguousarray(np.asarray(x, dtype="<f4"))
    codes = x.view(np.uint8).reshape(*x.shape[:-1], 4 * x.shape[-1])
    return codes, np.zeros((*x.shape[:-1], 0), np.float16)


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bytes uint8 [..., 4D] -> float32 [..., D]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return c.view("<f4").reshape(*c.shape[:-1], c.shape[-1] // 4).astype(np.float32)
