"""Build libkvq.so (HIP for gfx950) in place, next to this file, and the measurement library
libkvq_probe.so (a page-stream probe that bench.py times; libkvq does not use it).

    python -m quantized_paged_kv_kvq_amd.build [--asm]

The encoder and gather translation units are compiled with -ffp-contract=off so that every
binary32 product and sum rounds on its own (their output must equal the arithmetic contract
stated in include/kvq.h bit for bit).  Packed FP32 instructions are disabled for all HIP code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
PROBE_UNIT = "page_probe.hip"

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]
# translation unit -> extra flags.  The decode kernels need their page loops fully unrolled (a rolled
# loop waits for every outstanding load).  Their loops exit early after a wave's last page; the
# unroller's bound for fully unrolling such loops by their maximum trip count is 8 by default, and the
# 16-page loops of the ISO and q4_0 kernels (with their inline mixed-precision fmas) then stayed
# rolled for some instances (ISO3 at head_dim 256, 4 waves x 16 pages: 120.8 against 47.1 us for one
# sequence of 262,144 tokens), hence the bound of 16 for those units.  The k8v4 verify and q4_0-K
# kernels keep their MFMA accumulators in VGPRs (the default placed them in AGPRs and copied them
# around every MFMA).
UNITS = {
    "kvq_api.hip": [],
    "append.hip": ["-ffp-contract=off"],
    "gather.hip": ["-ffp-contract=off"],
    "decode.hip": ["-mllvm", "-pragma-unroll-threshold=200000", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode_verify.hip": ["-mllvm", "-pragma-unroll-threshold=200000", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode_iso.hip": ["-mllvm", "-pragma-unroll-threshold=200000", "-mllvm", "-unroll-max-upperbound=16"],
    "decode_q4.hip": ["-mllvm", "-pragma-unroll-threshold=200000", "-mllvm", "-unroll-max-upperbound=16",
                      "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode_f32.hip": ["-mllvm", "-pragma-unroll-threshold=200000", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "extend.hip": [],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(unit: str, extra, asm: bool) -> str:
    src = os.path.join(CSRC, unit)
    obj = os.path.join(BUILD, unit.replace(".hip", ".o"))
    cmd = [_hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {unit}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if asm:
        s = os.path.join(BUILD, unit.replace(".hip", f"-{ARCH}.s"))
        subprocess.run([_hipcc(), *COMMON, *extra, "--cuda-device-only", "-S", src, "-o", s],
                       capture_output=True, text=True, check=True)
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    units = [u for u in UNITS if os.path.exists(os.path.join(CSRC, u))]
    probe = [PROBE_UNIT] if os.path.exists(os.path.join(CSRC, PROBE_UNIT)) else []
    extra = {**UNITS, PROBE_UNIT: ["-mllvm", "-pragma-unroll-threshold=200000"]}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(units) + len(probe))) as ex:
        objs = list(ex.map(lambda u: _compile(u, extra[u], asm), units + probe))
    _link(objs[:len(units)], LIB)
    if probe:
        _link(objs[len(units):], PROBE_LIB)
    if verbose:
        print(f"built {LIB}" + (f" and {PROBE_LIB}" if probe else ""))
    return LIB


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


if __name__ == "__main__":
    build(asm="--asm" in sys.argv)
