"""CPU tests of the C-ABI library: it loads, exports every entry point include/kvq.h declares,
reports cell sizes that match the oracle, and refuses invalid arguments on the host before any
HIP call (so none of these need a GPU)."""
import ctypes
import os
import re

import pytest

from quantized_paged_kv_kvq_amd import kvq
from oracle import paged as opaged

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvq.h")
FAKE = 1 << 20          # a non-NULL, aligned pointer value that validation never dereferences


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    names = declared_functions()
    assert {"kvq_append", "kvq_decode_attn", "kvq_decode_attn_append", "kvq_extend_attn",
            "kvq_dequant_gather"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    ver = int(re.search(r"#define KVQ_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.kvq_abi_version() == ver


@pytest.mark.parametrize("fmt,D", [("int8", 64), ("int8", 128), ("int8", 256), ("int8", 512), ("q4h", 256),
                                   ("iso3", 128), ("iso3", 256), ("f32", 64), ("f32", 256), ("f32", 512),
                                   ("iso4", 128), ("iso4", 512)])
def test_cell_bytes_match_oracle(fmt, D):
    assert kvq.cell_bytes(fmt, D) == opaged.cell_bytes(fmt, D)


def test_cell_bytes_refuses_bad_geometry():
    L = kvq.lib()
    for fmt, D in ((1, 100), (2, 128), (3, 64), (9, 128), (1, 1024), (4, 96), (4, 1024), (5, 64), (5, 640)):
        assert L.kvq_cell_bytes(fmt, D, None, None) == -1


def make_cache(fk=1, fv=1, D=256, hkv=2, page=16, npages=64):
    c = kvq.KvqCache()
    c.n_kv_heads, c.head_dim, c.page_size, c.num_pages = hkv, D, page, npages
    c.k = kvq.KvqStore(fk, FAKE, FAKE)
    c.v = kvq.KvqStore(fv, FAKE, FAKE)
    return c


def make_pages(batch=1, max_pages=64):
    p = kvq.KvqPages()
    p.block_table, p.seq_lens, p.batch, p.max_pages = FAKE, FAKE, batch, max_pages
    return p


def decode(c, p, n_q=1, hq=16, head_map=None, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    L = kvq.lib()
    hm = None
    if head_map is not None:
        arr = (ctypes.c_int32 * len(head_map))(*head_map)
        hm = ctypes.cast(arr, ctypes.c_void_p)
    return L.kvq_decode_attn(ctypes.byref(c) if c else None, ctypes.byref(p) if p else None, q, n_q, hq, None, hm,
                             0.0625, out, ws, ws_bytes, None)


def test_decode_validation_errors():
    L = kvq.lib()
    assert decode(None, make_pages()) == 1
    assert decode(make_cache(), None) == 1
    assert decode(make_cache(page=8), make_pages()) == 3
    assert decode(make_cache(fk=2), make_pages()) == 3                 # q4_0 K needs a q4_0 V store
    assert decode(make_cache(fk=2, fv=2), make_pages(), n_q=3) == 3    # q4_0 K: 24 rows > 16
    assert decode(make_cache(fk=3, fv=1, D=128), make_pages()) == 3     # ISO3 K needs an ISO3 V store
    assert decode(make_cache(fk=1, fv=3, D=128), make_pages()) == 3     # and ISO3 V an ISO3 K store
    assert decode(make_cache(fk=3, fv=3, D=128), make_pages(), n_q=3) == 3    # ISO3: 24 rows > 16
    assert decode(make_cache(fk=3, fv=3, D=384), make_pages()) == 3     # ISO3 decode: head_dim 128 or 256
    assert decode(make_cache(D=100), make_pages()) == 3                 # int8 needs head_dim % 64
    assert decode(make_cache(fv=2, D=128), make_pages()) == 3           # Hadamard V needs 256
    assert decode(make_cache(), make_pages(), hq=15) == 2               # Hq % Hkv
    assert decode(make_cache(), make_pages(), hq=4, head_map=[0, 1, 2, 0]) == 2   # map out of range
    assert decode(make_cache(), make_pages(), n_q=5) == 3               # 5 * 8 rows > 32
    assert decode(make_cache(), make_pages(), n_q=0) == 2
    assert decode(make_cache(), make_pages(), q=None) == 1
    assert decode(make_cache(), make_pages(), q=FAKE + 2) == 2          # misaligned
    assert decode(make_cache(), make_pages(), ws=None) == 4
    assert decode(make_cache(), make_pages(), ws_bytes=16) == 4
    assert decode(make_cache(), make_pages(), ws=FAKE + 16) == 4       # needs 256-byte alignment
    assert decode(make_cache(), make_pages(batch=0)) == 2
    c = make_cache()
    c.v = kvq.KvqStore(1, None, FAKE)
    assert decode(c, make_pages()) == 1


def test_decode_validation_iso4():
    """ISO4 K and V: head_dim 128 or 256, up to 16 rows; no mixing with ISO3 or other stores."""
    assert decode(make_cache(fk=5, fv=3, D=128), make_pages()) == 3
    assert decode(make_cache(fk=3, fv=5, D=128), make_pages()) == 3
    assert decode(make_cache(fk=1, fv=5, D=128), make_pages()) == 3
    assert decode(make_cache(fk=5, fv=5, D=384), make_pages()) == 3
    assert decode(make_cache(fk=5, fv=5, D=128), make_pages(), n_q=3) == 3    # 24 rows > 16
    assert decode(make_cache(fk=5, fv=5, D=128), make_pages(), ws=None) == 4  # valid up to the workspace
    L = kvq.lib()
    c = make_cache(fk=5, fv=5, D=128)
    # one sequence, 2 KV heads: 128 splits of 64 pages fill the CUs once (one 8-wave workgroup each)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 8192, 1, 16, None) == 2 * 128 * 8 * (128 + 2) * 4
    # 64 splits of 64 pages would fill half of them -> 128 of 32
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 4096, 1, 16, None) == 2 * 128 * 8 * (128 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 2048, 1, 16, None) == 2 * 64 * 8 * (128 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 4, 8192, 1, 16, None) == 4 * 2 * 128 * 8 * (128 + 2) * 4


def test_decode_validation_single_store_modes():
    """k8v32 / k32v8 / F32 for both: head_dim 128 or 256, up to 32 rows, the other store int8; an
    F32 store needs no scales pointer."""
    assert decode(make_cache(fk=4, fv=2), make_pages()) == 3            # F32 K with q4_0 V
    assert decode(make_cache(fk=3, fv=4, D=128), make_pages()) == 3     # ISO3 K with F32 V
    assert decode(make_cache(fk=1, fv=4, D=64), make_pages(), hq=4) == 3    # head_dim 64
    assert decode(make_cache(fk=4, fv=1, D=512), make_pages(), hq=4) == 3   # head_dim 512
    assert decode(make_cache(fk=4, fv=1), make_pages(), n_q=5) == 3     # 40 rows > 32
    c = make_cache(fk=4, fv=4)
    c.k = kvq.KvqStore(4, FAKE, None)
    c.v = kvq.KvqStore(4, FAKE, None)
    assert decode(c, make_pages(), ws=None) == 4                        # reaches the workspace check
    c = make_cache(fk=1, fv=4)
    c.k = kvq.KvqStore(1, FAKE, None)                                   # int8 K still needs its scales
    assert decode(c, make_pages()) == 1


def decode_append(c, p, n_q=1, hq=16, k=FAKE, v=FAKE, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    L = kvq.lib()
    return L.kvq_decode_attn_append(ctypes.byref(c) if c else None, ctypes.byref(p) if p else None, k, v, q, n_q, hq,
                                    None, None, 0.0625, out, ws, ws_bytes, None)


def test_decode_append_validation_errors():
    assert decode_append(None, make_pages()) == 1
    assert decode_append(make_cache(fv=2, D=128), make_pages()) == 3    # q4_0 V: head_dim 256 only
    assert decode_append(make_cache(fk=2, fv=2), make_pages()) == 3     # fused path: int8 K only
    assert decode_append(make_cache(fk=3, fv=3, D=128), make_pages()) == 3   # no fused ISO3 step
    assert decode_append(make_cache(fk=4, fv=2), make_pages()) == 3     # F32 K with q4_0 V
    assert decode_append(make_cache(fk=3, fv=3, D=128), make_pages()) == 3
    assert decode_append(make_cache(), make_pages(), n_q=5, hq=4) == 3  # at most 4 new tokens per sequence
    assert decode_append(make_cache(), make_pages(), n_q=0) == 3
    assert decode_append(make_cache(), make_pages(), k=None) == 1
    assert decode_append(make_cache(), make_pages(), v=None) == 1
    assert decode_append(make_cache(), make_pages(), k=FAKE + 8) == 2   # misaligned
    assert decode_append(make_cache(), make_pages(), q=None) == 1       # then the decode checks
    assert decode_append(make_cache(), make_pages(), ws_bytes=16) == 4
    assert decode_append(make_cache(), None) == 1


def test_decode_workspace_size_formula():
    L = kvq.lib()
    c = make_cache()
    n = L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 8192, 1, 16, None)
    assert n == 2 * 128 * 8 * (256 + 2) * 4           # 2 KV heads x 128 splits x 8 rows x (D + m, l) fp32
    # 64-page splits fill at most about half of the CUs: the fewest pages per split (a multiple of 4, at
    # most 32) keeping one round (2,500 pages: 125 splits of 20); above that 64-page splits stay
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 2500, 1, 16, None) == 2 * 125 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 4096, 1, 16, None) == 2 * 128 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 7422, 1, 16, None) == 2 * 116 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(c), 1, 8192, 5, 16, None) == 0
    iso = make_cache(fk=3, fv=3, D=128)
    # ISO3 / ISO4 (like q4_0): 64-page splits while they fill more than half of the CUs
    assert L.kvq_decode_workspace_bytes(ctypes.byref(iso), 1, 8192, 1, 16, None) == 2 * 128 * 8 * (128 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(iso), 1, 8192, 2, 16, None) == 2 * 128 * 16 * (128 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(iso), 2, 8192, 1, 16, None) == 2 * 2 * 128 * 8 * (128 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(iso), 1, 8192, 3, 16, None) == 0
    for fk, fv in ((1, 4), (4, 1), (4, 4)):
        f = make_cache(fk=fk, fv=fv)
        assert L.kvq_decode_workspace_bytes(ctypes.byref(f), 1, 8192, 1, 16, None) == 2 * 128 * 8 * (256 + 2) * 4
        assert L.kvq_decode_workspace_bytes(ctypes.byref(f), 1, 8192, 3, 16, None) == 2 * 128 * 24 * (256 + 2) * 4
        assert L.kvq_decode_workspace_bytes(ctypes.byref(f), 1, 8192, 4, 16, None) == 2 * 128 * 32 * (256 + 2) * 4
        assert L.kvq_decode_workspace_bytes(ctypes.byref(f), 1, 8192, 5, 16, None) == 0
    # k8v4 verify (24 rows: the wave-pair kernel): the fewest pages per split (a multiple of 4, at most
    # 64) that keeps 2 KV heads within 256 workgroups
    k8v4 = make_cache(fk=1, fv=2)
    assert L.kvq_decode_workspace_bytes(ctypes.byref(k8v4), 1, 7422, 3, 16, None) == 2 * 124 * 24 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(k8v4), 1, 8192, 3, 16, None) == 2 * 128 * 24 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(k8v4), 1, 2000, 3, 16, None) == 2 * 125 * 24 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(k8v4), 1, 20000, 3, 16, None) == 2 * 313 * 24 * (256 + 2) * 4
    q4 = make_cache(fk=2, fv=2)
    # q4_0 the same
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 1, 8192, 1, 16, None) == 2 * 128 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 1, 8192, 2, 16, None) == 2 * 128 * 16 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 2, 8192, 1, 16, None) == 2 * 2 * 128 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 1, 4096, 1, 16, None) == 2 * 128 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 1, 2048, 1, 16, None) == 2 * 64 * 8 * (256 + 2) * 4
    assert L.kvq_decode_workspace_bytes(ctypes.byref(q4), 1, 8192, 3, 16, None) == 0


def test_append_and_gather_validation_errors():
    L = kvq.lib()
    c, p = make_cache(), make_pages()
    A = lambda c, p, k, v, n, ts=FAKE, tp=FAKE: L.kvq_append(ctypes.byref(c), ctypes.byref(p), k, v, ts, tp, n, None)
    assert A(c, p, FAKE, FAKE, -1) == 2
    assert A(c, p, FAKE, FAKE, 0) == 0                 # no-op, nothing launched
    assert A(c, p, None, None, 5) == 0
    assert A(c, p, FAKE, FAKE, 5, ts=None) == 1
    assert A(make_cache(fk=2, D=128), p, FAKE, None, 5) == 3   # q4_0 K store needs head_dim 256
    assert A(make_cache(page=32), p, FAKE, FAKE, 1) == 3
    assert A(make_cache(fk=4, fv=4, D=96), p, FAKE, FAKE, 1) == 3   # F32 store: head_dim % 64
    f = make_cache(fk=4, fv=4)
    f.k = kvq.KvqStore(4, FAKE + 8, None)
    assert A(f, p, FAKE, None, 1) == 2                 # misaligned codes
    G = lambda c, p, which, seq, start, count, dt=0, out=FAKE: L.kvq_dequant_gather(
        ctypes.byref(c), ctypes.byref(p), which, seq, start, count, dt, 0, out, None)
    assert G(c, p, 2, 0, 0, 1) == 2
    assert G(c, p, 0, 1, 0, 1) == 2                    # seq outside the batch
    assert G(c, p, 0, 0, 64 * 16 - 1, 2) == 2          # past the page table
    assert G(c, p, 0, 0, -1, 2) == 2
    assert G(c, p, 0, 0, 0, 1, dt=7) == 2
    assert G(c, p, 0, 0, 0, 1, out=None) == 1
    assert G(c, p, 0, 0, 0, 0) == 0
    assert L.kvq_status_str(3) == b"unsupported format or geometry"


def extend(c, p, n_new=64, max_new=64, hq=16, head_map=None, q=FAKE, kn=FAKE, vn=FAKE, cu=FAKE, out=FAKE,
           scale=0.0625):
    L = kvq.lib()
    hm = None
    if head_map is not None:
        arr = (ctypes.c_int32 * len(head_map))(*head_map)
        hm = ctypes.cast(arr, ctypes.c_void_p)
    return L.kvq_extend_attn(ctypes.byref(c) if c else None, ctypes.byref(p) if p else None, q, kn, vn, cu, n_new,
                             max_new, hq, hm, scale, out, 1, None, 0, None)


def test_extend_validation_errors():
    L = kvq.lib()
    iso = lambda **kw: make_cache(fk=3, fv=3, D=128, **kw)
    assert extend(None, make_pages()) == 1
    assert extend(iso(), None) == 1
    assert extend(make_cache(), make_pages()) == 3                      # int8 stores: head_dim 128 only
    assert extend(make_cache(D=128), make_pages(), cu=None) == 1        # int8 K and V at 128: accepted
    assert extend(make_cache(fk=1, fv=3, D=128), make_pages()) == 3     # mixed int8 / ISO3
    assert extend(make_cache(fk=4, fv=4, D=128), make_pages()) == 3     # F32 stores: no extend path
    assert extend(make_cache(fk=3, fv=3, D=256), make_pages()) == 3     # head_dim 128 only
    assert extend(iso(), make_pages(), max_new=65) == 2                 # max_new > n_new
    assert extend(iso(), make_pages(), n_new=-1, max_new=0) == 2
    assert extend(iso(), make_pages(), hq=15) == 2                      # Hq % Hkv
    assert extend(iso(hkv=1), make_pages(), hq=33) == 3                 # 33 query heads on one KV head
    assert extend(iso(), make_pages(), q=None) == 1
    assert extend(iso(), make_pages(), cu=None) == 1
    assert extend(iso(), make_pages(), kn=FAKE + 4) == 2                # misaligned
    assert extend(iso(), make_pages(), scale=float("nan")) == 2
    assert extend(iso(), make_pages(), n_new=0, max_new=0, q=None) == 0  # empty chunk: no-op
    c = iso()
    assert L.kvq_extend_workspace_bytes(ctypes.byref(c), 1, 64, 64, 64, 16) == 2 * (16 + 1) * 36864
    assert L.kvq_extend_workspace_bytes(ctypes.byref(make_cache()), 1, 64, 64, 64, 16) == 0
    i8 = make_cache(D=128)
    assert L.kvq_extend_workspace_bytes(ctypes.byref(i8), 1, 64, 64, 64, 16) == 2 * (16 + 1) * 36864


def decode_noalloc(c, p, n_q=1, hq=16, q=FAKE, out=FAKE):
    L = kvq.lib()
    return L.kvq_decode_attn_noalloc(ctypes.byref(c) if c else None, ctypes.byref(p) if p else None, q, n_q, hq,
                                     None, None, 0.0625, out, None)


def test_decode_noalloc_validation_and_scratch_limit():
    """kvq_decode_attn_noalloc validates like kvq_decode_attn, and refuses (on the host, before any HIP
    call) a call whose split partials exceed its fixed scratch, whose size the header states."""
    L = kvq.lib()
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == 16 << 20
    assert decode_noalloc(None, make_pages()) == 1
    assert decode_noalloc(make_cache(), make_pages(), n_q=5) == 3
    assert decode_noalloc(make_cache(), make_pages(), q=None) == 1
    c = make_cache(hkv=8, D=128)
    big = make_pages(batch=64, max_pages=4096)
    need = L.kvq_decode_workspace_bytes(ctypes.byref(c), 64, 4096, 1, 32, None)
    assert need > limit
    assert decode_noalloc(c, big, hq=32) == 4
    assert "scratch" in L.kvq_last_error().decode()
