"""Python binding of libkvq (ctypes).  Argument marshalling only: every step of the hot path
runs in the HIP kernels behind the C ABI declared in include/kvq.h, and each function here has
the name of the entry point it calls.  PyTorch provides device memory and streams.

There is no fallback: if libkvq.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

FMT = {"int8": 1, "q4h": 2, "iso3": 3, "f32": 4, "iso4": 5}
OUT_DTYPE = {"f32": (0, torch.float32), "f16": (1, torch.float16), "bf16": (2, torch.bfloat16)}
PAGE_SIZE = 16

STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_NULL", 2: "KVQ_ERR_SHAPE", 3: "KVQ_ERR_UNSUPPORTED",
          4: "KVQ_ERR_WORKSPACE", 5: "KVQ_ERR_HIP"}


class KVQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class KvqStore(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("codes", c_void_p), ("scales", c_void_p)]


class KvqCache(ctypes.Structure):
    _fields_ = [("n_kv_heads", c_int32), ("head_dim", c_int32), ("page_size", c_int32), ("num_pages", c_int32),
                ("k", KvqStore), ("v", KvqStore), ("iso_quat", c_float * 4)]


class KvqPages(ctypes.Structure):
    _fields_ = [("block_table", c_void_p), ("seq_lens", c_void_p), ("batch", c_int32), ("max_pages", c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built in place by quantized_paged_kv_kvq_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m quantized_paged_kv_kvq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        cp, ip = POINTER(KvqCache), POINTER(KvqPages)
        L.kvq_append.argtypes = [cp, ip, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]
        L.kvq_decode_attn.argtypes = [cp, ip, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_float, c_void_p,
                                      c_void_p, c_size_t, c_void_p]
        L.kvq_decode_attn_append.argtypes = [cp, ip, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                             c_void_p, c_float, c_void_p, c_void_p, c_size_t, c_void_p]
        L.kvq_decode_attn_noalloc.argtypes = [cp, ip, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_float,
                                              c_void_p, c_void_p]
        L.kvq_decode_workspace_bytes.argtypes = [cp, c_int32, c_int32, c_int32, c_int32, c_void_p]
        L.kvq_decode_workspace_bytes.restype = c_size_t
        L.kvq_extend_attn.argtypes = [cp, ip, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                      c_void_p, c_float, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]
        L.kvq_extend_workspace_bytes.argtypes = [cp, c_int32, c_int32, c_int32, c_int32, c_int32]
        L.kvq_extend_workspace_bytes.restype = c_size_t
        L.kvq_dequant_gather.argtypes = [cp, ip, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p]
        L.kvq_cell_bytes.argtypes = [c_int32, c_int32, POINTER(c_int32), POINTER(c_int32)]
        L.kvq_cell_bytes.restype = c_int32
        L.kvq_status_str.argtypes = [c_int32]
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_last_error.restype = ctypes.c_char_p
        L.kvq_abi_version.restype = c_int32
        for name in ("kvq_append", "kvq_decode_attn", "kvq_decode_attn_append", "kvq_decode_attn_noalloc",
                     "kvq_extend_attn", "kvq_dequant_gather"):
            getattr(L, name).restype = c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise KVQError(status, lib().kvq_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype, device: torch.device, optional: bool = False):
    """Raise ValueError / TypeError unless t has this shape, dtype and device (checked before any launch:
    the kernels trust these sizes, so a mismatch would read or write past a buffer on the device)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _expect_numel(t: Optional[torch.Tensor], name: str, n: int, dtype, device: torch.device, optional: bool = False):
    """As _expect for index arrays whose element count matters, not their shape."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _on_gpu(dev: torch.device):
    if dev.type != "cuda":
        raise ValueError(f"the cache slabs must be on a GPU, got {dev} (the kernels take device pointers only)")


def _head_map_len(head_map, n_q_heads: int):
    if head_map is not None and len(head_map) != n_q_heads:
        raise ValueError(f"head_map must have one entry per query head ({n_q_heads}), got {len(head_map)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def cell_bytes(fmt: str, head_dim: int):
    """(code bytes, fp16 scale count) of one (token, KV head) cell of one store."""
    cb, ns = c_int32(), c_int32()
    if lib().kvq_cell_bytes(FMT[fmt], head_dim, ctypes.byref(cb), ctypes.byref(ns)) < 0:
        raise KVQError(3, f"format {fmt} does not support head_dim {head_dim}")
    return cb.value, ns.value


class PagedKVCache:
    """Device slabs of a paged quantised KV cache (owned here as torch tensors) and their descriptor.

    codes:  uint8  [num_pages][n_kv_heads][page_size * code_bytes]  (byte order per include/kvq.h)
    scales: fp16   [num_pages][n_kv_heads][page_size][n_scales]
    """

    def __init__(self, num_pages: int, n_kv_heads: int, head_dim: int, fmt_k: str = "int8", fmt_v: str = "int8",
                 device="cuda", quat: Sequence[float] = (1.0, 0.0, 0.0, 0.0)):
        self.num_pages, self.n_kv_heads, self.head_dim = num_pages, n_kv_heads, head_dim
        self.fmt_k, self.fmt_v = fmt_k, fmt_v
        self.quat = [float(x) for x in quat]
        cbk, nsk = cell_bytes(fmt_k, head_dim)
        cbv, nsv = cell_bytes(fmt_v, head_dim)
        self.k_codes = torch.zeros((num_pages, n_kv_heads, PAGE_SIZE * cbk), dtype=torch.uint8, device=device)
        self.k_scales = torch.zeros((num_pages, n_kv_heads, PAGE_SIZE, nsk), dtype=torch.float16, device=device)
        self.v_codes = torch.zeros((num_pages, n_kv_heads, PAGE_SIZE * cbv), dtype=torch.uint8, device=device)
        self.v_scales = torch.zeros((num_pages, n_kv_heads, PAGE_SIZE, nsv), dtype=torch.float16, device=device)
        self._desc = None

    @property
    def device(self) -> torch.device:
        return self.k_codes.device

    def descriptor(self) -> KvqCache:
        if self._desc is None:
            d = KvqCache()
            d.n_kv_heads, d.head_dim, d.page_size, d.num_pages = (self.n_kv_heads, self.head_dim, PAGE_SIZE,
                                                                  self.num_pages)
            d.k = KvqStore(FMT[self.fmt_k], self.k_codes.data_ptr(), self.k_scales.data_ptr())
            d.v = KvqStore(FMT[self.fmt_v], self.v_codes.data_ptr(), self.v_scales.data_ptr())
            d.iso_quat = (c_float * 4)(*self.quat)
            self._desc = d
        return self._desc


class Pages:
    """Page table int32 [batch][max_pages] and lengths int32 [batch], both on the device."""

    def __init__(self, block_table: torch.Tensor, seq_lens: torch.Tensor):
        if block_table.dim() != 2:
            raise ValueError("block_table must be [batch][max_pages]")
        if seq_lens.numel() != block_table.shape[0]:
            raise ValueError(f"seq_lens must have one entry per sequence ({block_table.shape[0]}), "
                             f"got {seq_lens.numel()}")
        if seq_lens.device != block_table.device:
            raise ValueError("block_table and seq_lens must be on the same device")
        self.block_table, self.seq_lens = block_table, seq_lens
        d = KvqPages()
        d.block_table = _ptr(block_table, torch.int32, "block_table")
        d.seq_lens = _ptr(seq_lens, torch.int32, "seq_lens")
        d.batch, d.max_pages = block_table.shape[0], block_table.shape[1]
        self._desc = d

    @property
    def batch(self) -> int:
        return self._desc.batch

    @property
    def max_pages(self) -> int:
        return self._desc.max_pages

    @property
    def device(self) -> torch.device:
        return self.block_table.device

    def descriptor(self) -> KvqPages:
        return self._desc


def _head_map_arg(head_map):
    if head_map is None:
        return None, None
    arr = (c_int32 * len(head_map))(*[int(h) for h in head_map])
    return arr, ctypes.cast(arr, c_void_p)


def kvq_append(cache: PagedKVCache, pages: Pages, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
               tok_seq: torch.Tensor, tok_pos: torch.Tensor, stream=None) -> None:
    """Quantise bf16 [n_tok][n_kv_heads][head_dim] K and/or V into the cells (tok_seq[i], tok_pos[i])."""
    n_tok = tok_seq.numel()
    dev = cache.device
    _expect_numel(tok_seq, "tok_seq", n_tok, torch.int32, dev)
    _expect_numel(tok_pos, "tok_pos", n_tok, torch.int32, dev)
    shape = (n_tok, cache.n_kv_heads, cache.head_dim)
    _expect(k_new, "k_new", shape, torch.bfloat16, dev, optional=True)
    _expect(v_new, "v_new", shape, torch.bfloat16, dev, optional=True)
    if pages.device != dev:
        raise ValueError(f"the page table must be on {dev}, got {pages.device}")
    _on_gpu(dev)
    _check(lib().kvq_append(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                            _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
                            _ptr(tok_seq, torch.int32, "tok_seq"), _ptr(tok_pos, torch.int32, "tok_pos"),
                            n_tok, _stream(stream)))


def kvq_decode_workspace_bytes(cache: PagedKVCache, batch: int, max_pages: int, n_q: int, n_q_heads: int,
                               head_map=None) -> int:
    keep, hm = _head_map_arg(head_map)
    n = lib().kvq_decode_workspace_bytes(ctypes.byref(cache.descriptor()), batch, max_pages, n_q, n_q_heads, hm)
    del keep
    if n == 0:
        raise KVQError(2, lib().kvq_last_error().decode())
    return n


def _decode_shapes(cache: PagedKVCache, pages: Pages, q: torch.Tensor, q_lens, head_map, out):
    """Check the decode tensors against the cache and page-table descriptors; (B, n_q, Hq, D)."""
    dev = cache.device
    if q.dim() != 4:
        raise ValueError(f"q must be [batch][n_q][n_q_heads][head_dim], got shape {tuple(q.shape)}")
    B, n_q, Hq, D = q.shape
    _expect(q, "q", (pages.batch, n_q, Hq, cache.head_dim), torch.bfloat16, dev)
    if pages.device != dev:
        raise ValueError(f"the page table must be on {dev}, got {pages.device}")
    _expect_numel(q_lens, "q_lens", B * n_q, torch.int32, dev, optional=True)
    _expect(out, "out", (B, n_q, Hq, D), torch.float32, dev, optional=True)
    _head_map_len(head_map, Hq)
    return B, n_q, Hq, D


def kvq_decode_attn(cache: PagedKVCache, pages: Pages, q: torch.Tensor, q_lens: Optional[torch.Tensor] = None,
                    head_map=None, sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode / verify attention.  q: bf16 [batch][n_q][n_q_heads][head_dim] -> fp32 of the same shape."""
    B, n_q, Hq, D = _decode_shapes(cache, pages, q, q_lens, head_map, out)
    _on_gpu(cache.device)
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = kvq_decode_workspace_bytes(cache, pages.batch, pages.max_pages, n_q, Hq, head_map)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    keep, hm = _head_map_arg(head_map)
    _check(lib().kvq_decode_attn(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                                 _ptr(q, torch.bfloat16, "q"), n_q, Hq, _ptr(q_lens, torch.int32, "q_lens"), hm,
                                 float(sm_scale), _ptr(out, torch.float32, "out"), _ptr(workspace, None, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    del keep
    return out


def kvq_decode_attn_noalloc(cache: PagedKVCache, pages: Pages, q: torch.Tensor, q_lens: Optional[torch.Tensor] = None,
                            head_map=None, sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """kvq_decode_attn without a workspace: the split partials go to the library's own per-GPU scratch
    (calls that overlap in time on one GPU race).  `out` must be passed by callers that cannot allocate."""
    B, n_q, Hq, D = _decode_shapes(cache, pages, q, q_lens, head_map, out)
    _on_gpu(cache.device)
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device=q.device)
    keep, hm = _head_map_arg(head_map)
    _check(lib().kvq_decode_attn_noalloc(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                                         _ptr(q, torch.bfloat16, "q"), n_q, Hq, _ptr(q_lens, torch.int32, "q_lens"),
                                         hm, float(sm_scale), _ptr(out, torch.float32, "out"), _stream(stream)))
    del keep
    return out


def kvq_decode_attn_append(cache: PagedKVCache, pages: Pages, k_new: torch.Tensor, v_new: torch.Tensor,
                           q: torch.Tensor, q_lens: Optional[torch.Tensor] = None, head_map=None,
                           sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode step in one launch: k/v_new bf16 [batch][n_q][n_kv_heads][head_dim] go to positions
    seq_lens[b] - n_q .. seq_lens[b] - 1, then attention as kvq_decode_attn."""
    B, n_q, Hq, D = _decode_shapes(cache, pages, q, q_lens, head_map, out)
    _expect(k_new, "k_new", (B, n_q, cache.n_kv_heads, D), torch.bfloat16, cache.device)
    _expect(v_new, "v_new", (B, n_q, cache.n_kv_heads, D), torch.bfloat16, cache.device)
    _on_gpu(cache.device)
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = kvq_decode_workspace_bytes(cache, pages.batch, pages.max_pages, n_q, Hq, head_map)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    keep, hm = _head_map_arg(head_map)
    _check(lib().kvq_decode_attn_append(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                                        _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
                                        _ptr(q, torch.bfloat16, "q"), n_q, Hq, _ptr(q_lens, torch.int32, "q_lens"),
                                        hm, float(sm_scale), _ptr(out, torch.float32, "out"),
                                        _ptr(workspace, None, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    del keep
    return out


def kvq_extend_workspace_bytes(cache: PagedKVCache, batch: int, max_pages: int, n_new: int, max_new: int,
                               n_q_heads: int) -> int:
    return int(lib().kvq_extend_workspace_bytes(ctypes.byref(cache.descriptor()), batch, max_pages, n_new, max_new,
                                                n_q_heads))


def kvq_extend_attn(cache: PagedKVCache, pages: Pages, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    cu_new: torch.Tensor, max_new: int, head_map=None, sm_scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, pack_after: bool = True,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Extend (prefill chunk) attention.  q: bf16 [n_new][n_q_heads][D]; k/v_new: bf16 [n_new][n_kv_heads][D]."""
    dev = cache.device
    if q.dim() != 3:
        raise ValueError(f"q must be [n_new][n_q_heads][head_dim], got shape {tuple(q.shape)}")
    N, Hq, D = q.shape
    _expect(q, "q", (N, Hq, cache.head_dim), torch.bfloat16, dev)
    _expect(k_new, "k_new", (N, cache.n_kv_heads, cache.head_dim), torch.bfloat16, dev)
    _expect(v_new, "v_new", (N, cache.n_kv_heads, cache.head_dim), torch.bfloat16, dev)
    _expect_numel(cu_new, "cu_new", pages.batch + 1, torch.int32, dev)
    _expect(out, "out", (N, Hq, D), torch.float32, dev, optional=True)
    if pages.device != dev:
        raise ValueError(f"the page table must be on {dev}, got {pages.device}")
    _head_map_len(head_map, Hq)
    _on_gpu(dev)
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = kvq_extend_workspace_bytes(cache, pages.batch, pages.max_pages, N, max_new, Hq)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    keep, hm = _head_map_arg(head_map)
    _check(lib().kvq_extend_attn(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                                 _ptr(q, torch.bfloat16, "q"), _ptr(k_new, torch.bfloat16, "k_new"),
                                 _ptr(v_new, torch.bfloat16, "v_new"), _ptr(cu_new, torch.int32, "cu_new"), N,
                                 int(max_new), Hq, hm, float(sm_scale), _ptr(out, torch.float32, "out"),
                                 1 if pack_after else 0, _ptr(workspace, None, "workspace"), ws_bytes,
                                 _stream(stream)))
    del keep
    return out


def kvq_dequant_gather(cache: PagedKVCache, pages: Pages, which: str, seq: int, start: int, count: int,
                       out_dtype: str = "f32", unrotate: bool = False, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Dequantised cells [start, start+count) of sequence `seq`: [count][n_kv_heads][head_dim]."""
    code, tdt = OUT_DTYPE[out_dtype]
    _expect(out, "out", (count, cache.n_kv_heads, cache.head_dim), tdt, cache.device, optional=True)
    if pages.device != cache.device:
        raise ValueError(f"the page table must be on {cache.device}, got {pages.device}")
    _on_gpu(cache.device)
    if out is None:
        out = torch.empty((count, cache.n_kv_heads, cache.head_dim), dtype=tdt, device=cache.k_codes.device)
    _check(lib().kvq_dequant_gather(ctypes.byref(cache.descriptor()), ctypes.byref(pages.descriptor()),
                                    {"k": 0, "v": 1}[which], seq, start, count, code, 1 if unrotate else 0,
                                    _ptr(out, tdt, "out"), _stream(stream)))
    return out
