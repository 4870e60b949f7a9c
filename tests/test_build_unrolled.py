"""The built library's decode kernels have fully unrolled page loops (runs without a GPU).

A decode kernel's page loop must be straight-line code: rolled, its register ring of pages is indexed
at run time and every wait on the vector memory counter covers all outstanding loads (an ISO3
head_dim-256 instance that stayed rolled ran 2.6x slower).  Each kernel template is instantiated for
several pages per wave (PPW); with the loop unrolled, its matrix instructions grow in proportion to
PPW within a family of otherwise equal template arguments.  The check disassembles the gfx950 code
objects of libkvq.so (built here) with llvm-objdump.
"""
import collections
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_paged_kv_kvq_amd", "libkvq.so")
LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# kernel template -> index of its pages-per-wave argument
PPW_ARG = {"k_decode_split": 4, "k_decode_q4": 2, "k_decode_iso": 4, "k_decode_f32": 5, "k_verify_k8v4": 1}


def _code_objects(tmp_path):
    """The gfx950 code objects of the library's offload bundles (one per translation unit)."""
    fat = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", LIB,
                    str(tmp_path / "lib.so")], check=True, capture_output=True)
    data = fat.read_bytes()
    out = []
    for m in re.finditer(re.escape(BUNDLE_MAGIC), data):
        s = m.start()
        p = s + len(BUNDLE_MAGIC)
        (n,) = struct.unpack_from("<Q", data, p)
        p += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if "gfx950" in triple and size:
                out.append(data[s + off:s + off + size])
    return out


def _mfma_counts(tmp_path):
    counts = collections.Counter()
    for i, co in enumerate(_code_objects(tmp_path)):
        f = tmp_path / f"co{i}.o"
        f.write_bytes(co)
        text = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", "-C", str(f)],
                              check=True, capture_output=True, text=True).stdout
        name = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.*)>:$", line)
            if m:
                name = m.group(1)
            elif name and "v_mfma" in line:
                counts[name] += 1
    return counts


@pytest.mark.skipif(not (os.path.exists(LIB) and shutil.which(os.path.join(LLVM, "llvm-objdump"))),
                    reason="libkvq.so or the ROCm LLVM tools are missing")
def test_decode_page_loops_unrolled(tmp_path):
    families = collections.defaultdict(list)
    for name, n in _mfma_counts(tmp_path).items():
        m = re.search(r"(k_decode_split|k_decode_q4|k_decode_iso|k_decode_f32|k_verify_k8v4)<([^>]*)>", name)
        if not m:
            continue
        args = [x.strip() for x in m.group(2).split(",")]
        ppw = int(args[PPW_ARG[m.group(1)]])
        # the family: every template argument but the launch shape (waves, pages per wave, pages in
        # flight, occupancy), which only changes the page loop's trip count
        shape_free = tuple(a for i, a in enumerate(args) if i != PPW_ARG[m.group(1)] and not (
            m.group(1) != "k_verify_k8v4" and i in _shape_args(m.group(1))))
        families[(m.group(1), shape_free)].append((ppw, n, m.group(0)))
    assert sum(len(v) for v in families.values()) >= 40, "decode kernels not found in the code objects"
    for key, inst in families.items():
        # the matrix instructions of these kernels all sit in the page loop, so an unrolled instance
        # has PPW times one page's worth; a rolled one has one page's worth whatever its PPW
        per_page = max(n / ppw for ppw, n, _ in inst)
        for ppw, n, kernel in inst:
            assert n >= ppw * per_page * 0.99, f"{kernel}: {n} MFMAs for {ppw} pages per wave (rolled page loop?)"


def _shape_args(kernel):
    """Indices of the launch-shape template arguments other than pages per wave."""
    return {"k_decode_split": {3, 5, 6}, "k_decode_q4": {1, 3, 4}, "k_decode_iso": {3, 5, 6},
            "k_decode_f32": {4, 6}}[kernel]
