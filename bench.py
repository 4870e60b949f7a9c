"""Benchmark of the quantized paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the hot path over the workload: quantize-on-write of the step's new K/V
tokens into the paged cache and decode (or MTP-verify) attention over the whole context -- one
fused launch sequence for int8 K and V (the decode kernel encodes the step's cells), otherwise an
append launch followed by the decode (--unfused forces the latter).
Default workload: one full-attention layer of a Qwen3.5-MoE-style model with int8 group-64 K and
V at 131,072 tokens of context (GQA 16:2, head_dim 256, page size 16, seeded random page
table).  Inputs are resident in HBM before the timed region.  The cache is replicated so that
consecutive steps read different copies whose total exceeds the 256 MB last-level (Infinity)
cache: every step streams its codes and scales from HBM.

Prints ONE JSON line.  `value` is microseconds per step (lower is better); `roofline` reports
the decode attention launch (fused or plain split-K kernel + log-sum-exp combine, timed with HIP
events on the stream it runs on, around batches of back-to-back launches) against the 8 TB/s HBM
peak on its algorithmic bytes; `cpu_baseline` times the CPU oracle on a bounded sample of the
same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0        # dense fp16 / bf16 matrix peak of MI355X
MALL_BYTES = 256 << 20
METRIC = "decode-attn µs/step + achieved HBM GB/s vs peak, int8 KV @128K ctx"
EXTEND_METRIC = "extend-attn µs/step + achieved MFMA TFLOP/s vs dense fp16 peak, ISO3 KV, 30k prefix + 2048 new"


def make_workload(name: str, ctx: int = 0):
    """The named workload; ctx > 0 sets the context of the single-sequence MoE-layer decode workloads."""
    import synth
    if ctx and name.startswith("moe_") and name != "moe_int8_decode_64k":
        if name == "moe_int8_decode":
            return synth.moe_int8_decode(ctx=ctx)
        if name in ("moe_iso3_decode", "moe_iso4_decode"):
            return synth.moe_iso3_decode(ctx=ctx, fmt=name[4:8])
        if name == "moe_q4h_decode":
            return synth.moe_q4h_decode(ctx=ctx)
        if name in ("moe_k8v32_decode", "moe_k32v8_decode"):
            return synth.moe_single_store_decode("int8" if name[5] == "8" else "f32",
                                                 "f32" if name[5] == "8" else "int8", ctx=ctx)
    elif ctx:
        raise SystemExit("--ctx applies to the single-sequence moe_* decode workloads")
    if name == "moe_int8_decode":
        return synth.moe_int8_decode(ctx=131072)
    if name == "moe_int8_decode_64k":
        return synth.moe_int8_decode(ctx=65536)
    if name == "k8v4_verify":
        return synth.k8v4_verify()
    if name == "batched_int8_decode":
        return synth.batched_int8_decode()
    if name == "tiny_int8_decode":
        return synth.tiny_int8_decode()
    if name == "iso3_extend":
        return synth.iso3_extend()
    if name == "int8_extend":
        return synth.iso3_extend(fmt="int8")
    if name == "batched_iso3_decode":
        return synth.batched_iso3_decode()
    if name == "moe_iso3_decode":
        return synth.moe_iso3_decode(ctx=131072)
    if name == "moe_q4h_decode":
        return synth.moe_q4h_decode(ctx=131072)
    if name == "moe_iso4_decode":
        return synth.moe_iso3_decode(ctx=131072, fmt="iso4")
    if name == "moe_k8v32_decode":
        return synth.moe_single_store_decode("int8", "f32", ctx=131072)
    if name == "moe_k32v8_decode":
        return synth.moe_single_store_decode("f32", "int8", ctx=131072)
    raise SystemExit(f"unknown workload {name}")


def algorithmic_bytes(w, cb_k, ns_k, cb_v, ns_v, fused=False):
    """Bytes one decode launch must move: every visible cell's codes and scales, the page-table
    entries it walks, q in, out; fused with quantize-on-write also the step's bf16 K/V in and its
    cells' codes and scales out."""
    cells = int(np.sum(np.maximum(w.seq_lens, 0)))
    per_cell = w.n_kv_heads * ((cb_k + 2 * ns_k) + (cb_v + 2 * ns_v))
    pages = int(np.sum((w.seq_lens + w.page_size - 1) // w.page_size))
    q = w.batch * w.n_q * w.n_q_heads * w.head_dim * 2
    out = w.batch * w.n_q * w.n_q_heads * w.head_dim * 4
    new = w.batch * w.n_step * (2 * w.n_kv_heads * w.head_dim * 2 + per_cell) if fused else 0
    return cells * per_cell + pages * 4 + q + out + new


def fusable(w):
    """The step can run as one fused quantize-on-write + decode launch sequence."""
    plain = w.fmt_k in ("int8", "f32") and w.fmt_v in ("int8", "f32")
    k8v4 = w.fmt_k == "int8" and w.fmt_v == "q4h" and w.head_dim == 256
    return (plain or k8v4) and w.n_step == w.n_q and 1 <= w.n_q <= 4


def recorded_traffic(workload: str):
    """HBM bytes per decode launch from the committed FETCH_SIZE / WRITE_SIZE profile of this workload,
    or None when there is none or the decode kernel source has changed since it was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "decode_int8_moe_131072.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"traffic-record: workload=(\S+) source=(\S+) source_sha256_16=([0-9a-f]+) traffic_bytes=(\d+)",
                  open(path).read())
    if not m or m.group(1) != workload:
        return None
    src = os.path.join(ROOT, m.group(2))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != m.group(3):
        return None
    return int(m.group(4))


def recorded_kernel(workload: str):
    """The split kernel's cold median (us) from the committed kernel-trace record of this workload, or
    None when there is none or the decode kernel source has changed since the trace was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "decode_int8_moe_131072.md")
    if not os.path.exists(path):
        return None
    for m in re.finditer(r"kernel-record: workload=(\S+) kernel=(\S+) source=(\S+) source_sha256_16=([0-9a-f]+) "
                         r"median_us=([0-9.]+)", open(path).read()):
        if m.group(1) != workload:
            continue
        src = os.path.join(ROOT, m.group(3))
        if os.path.exists(src) and hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] == m.group(4):
            return {"kernel": m.group(2), "median_us": float(m.group(5))}
    return None


def host_info():
    """CPU model, the machine's physical cores and the threads this process may run on."""
    model, cores, phys, core = None, set(), None, None
    try:
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and model is None:
                model = val
            elif key == "physical id":
                phys = val
            elif key == "core id":
                core = val
            elif not key and phys is not None:
                cores.add((phys, core))
                phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(cores) or None, "usable_threads": usable}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline(w, budget_s: float = 15.0, gpu_out=None, gpu_cache=None):
    """Time the oracle's step (encode the step's tokens, then fp64 attention over the dequantised
    cache) on the host cores -- all the threads its BLAS pool has, then one thread -- with the
    oracle's cache filled first, outside the timing.  Returns (baseline, parity): the parity verdict
    of the GPU step's output and cache slabs against the oracle's (when they are passed in)."""
    from oracle import attention as oatt
    from oracle import paged as opaged
    threads = blas_threads()
    sk = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = opaged.Store.empty(w.fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    for b in range(w.batch):
        P = int(w.seq_lens[b]) - w.n_step
        opaged.append(sk, w.block_table, np.full(P, b), np.arange(P), w.k[b][:P], w.page_size, quat=w.quat)
        opaged.append(sv, w.block_table, np.full(P, b), np.arange(P), w.v[b][:P], w.page_size, quat=w.quat)

    def step():
        for b in range(w.batch):
            L = int(w.seq_lens[b])
            pos = np.arange(L - w.n_step, L)
            opaged.append(sk, w.block_table, np.full(w.n_step, b), pos, w.k[b][L - w.n_step:], w.page_size, quat=w.quat)
            opaged.append(sv, w.block_table, np.full(w.n_step, b), pos, w.v[b][L - w.n_step:], w.page_size, quat=w.quat)
        return oatt.decode(sk, sv, w.block_table, w.seq_lens, w.q, w.page_size, w.sm_scale, q_lens=w.q_lens,
                           quat=w.quat)

    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ref = step()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s or len(times) >= 20:
            break
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            t0 = time.perf_counter()
            step()
            one = time.perf_counter() - t0
    except ImportError:
        pass
    per_step = float(np.median(times))
    base = {"value": per_step * 1e6, "unit": "us/step", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full steps of the same workload (median); numpy fp32 encode of the "
                      f"step's tokens + fp64 attention over all {int(np.sum(w.seq_lens))} cells",
            "value_1thread": round(one * 1e6, 1) if one is not None else None, **host_info()}
    parity = None
    if gpu_out is not None:
        parity = parity_verdict(w, sk, sv, ref, gpu_out, gpu_cache)
    return base, parity


def parity_verdict(w, sk, sv, ref, gpu_out, gpu_cache):
    """The benched step against the oracle, computed outside the timed region: attention errors over
    every output element and row, and byte mismatches of every cell of both stores (codes and scales)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kvq_testutil import attention_errors, gpu_slabs_token_major
    maxabs, cos, row_cos = attention_errors(gpu_out, ref)
    code_bad = scale_bad = 0
    for which, st in (("k", sk), ("v", sv)):
        codes, scales = gpu_slabs_token_major(gpu_cache, which)
        code_bad += int(np.count_nonzero(codes != st.codes))
        scale_bad += int(np.count_nonzero(scales.view(np.uint16) != st.scales.view(np.uint16)))
    ok = maxabs <= 1e-3 and cos > 0.9999 and row_cos > 0.9999 and code_bad == 0 and scale_bad == 0
    return {"max_abs": float(f"{maxabs:.3e}"), "cosine": round(cos, 9), "min_row_cosine": round(row_cos, 9),
            "code_byte_mismatches": code_bad, "scale_mismatches": scale_bad,
            "cells_checked": int(np.sum(w.seq_lens)) * w.n_kv_heads * 2, "pass": bool(ok),
            "bar": "max-abs <= 1e-3, cosine and min row cosine > 0.9999, codes and scales byte-identical"}


def extend_flops(w):
    """Algorithmic flops of one extend launch: QK and PV over every (row, visible key) pair."""
    pre, new = w.prefix_lens(), w.new_lens()
    keys = sum(int(new[b]) * int(pre[b]) + int(new[b]) * (int(new[b]) + 1) // 2 for b in range(w.batch))
    return 4.0 * keys * w.n_q_heads * w.head_dim


def extend_cpu_baseline(w, budget_s: float = 15.0):
    """The oracle's extend on a sample of query rows, scaled to the whole chunk, plus its encode of
    the chunk's tokens (deferred packing); the oracle's prefix is encoded first, outside the timing."""
    from oracle import attention as oatt
    from oracle import paged as opaged
    threads = blas_threads()
    pre, new = w.prefix_lens(), w.new_lens()
    P, N = int(pre[0]), int(new[0])
    sk = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = opaged.Store.empty(w.fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    opaged.append(sk, w.block_table, np.zeros(P, int), np.arange(P), w.k[0][:P], w.page_size, quat=w.quat)
    opaged.append(sv, w.block_table, np.zeros(P, int), np.arange(P), w.v[0][:P], w.page_size, quat=w.quat)
    cu = np.array([0, N], np.int32)
    rows = np.linspace(0, N - 1, 16).astype(np.int64)
    t0 = time.perf_counter()
    n_calls = 0
    while True:
        oatt.extend(sk, sv, w.block_table, pre, w.q, w.k[0][P:], w.v[0][P:], cu, w.page_size, w.sm_scale,
                    quat=w.quat, rows=rows)
        n_calls += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    t_rows = (time.perf_counter() - t0) / n_calls
    t1 = time.perf_counter()
    sk2 = opaged.Store.empty(w.fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    opaged.append(sk2, w.block_table, np.zeros(N, int), np.arange(P, P + N), w.k[0][P:], w.page_size, quat=w.quat)
    opaged.append(sk2, w.block_table, np.zeros(N, int), np.arange(P, P + N), w.v[0][P:], w.page_size, quat=w.quat)
    t_pack = time.perf_counter() - t1
    per_step = t_rows * N / len(rows) + t_pack
    return {"value": per_step * 1e6, "unit": "us/step", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 attention of {len(rows)} of {N} query tokens (all {w.n_q_heads} heads, "
                      f"{n_calls} runs) scaled by {N}/{len(rows)}, plus the numpy encode of the {N} new tokens",
            **host_info()}


def bench_extend(args):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    from synth import dev_bf16, dev_i32

    w = make_workload(args.workload)
    pre, new = w.prefix_lens(), w.new_lens()
    P, N = int(pre[0]), int(new[0])
    cache = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
    pages = kvq.Pages(dev_i32(w.block_table), dev_i32(pre))
    kvq.kvq_append(cache, pages, dev_bf16(w.k[0][:P]), dev_bf16(w.v[0][:P]), dev_i32(np.zeros(P, np.int32)),
                   dev_i32(np.arange(P, dtype=np.int32)))
    q, kn, vn = dev_bf16(w.q), dev_bf16(w.k[0][P:]), dev_bf16(w.v[0][P:])
    cu = dev_i32(np.array([0, N], np.int32))
    out = torch.empty((N, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(pack, stream):
        kvq.kvq_extend_attn(cache, pages, q, kn, vn, cu, N, sm_scale=w.sm_scale, out=out, pack_after=pack,
                            stream=stream)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(True, stream)
    torch.cuda.synchronize()
    mode = "eager"
    g_step = g_att = None
    if not args.no_graph:
        try:
            g_step, g_att = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_step):
                step(True, torch.cuda.current_stream())
            with torch.cuda.graph(g_att):
                step(False, torch.cuda.current_stream())
            g_step.replay(); g_att.replay()
            torch.cuda.synchronize()
            mode = "hip-graph"
        except Exception as e:  # noqa: BLE001
            print(f"[bench] graph capture unavailable ({e}); timing eager launches", file=sys.stderr, flush=True)
            g_step = g_att = None
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g_step.replay() if g_step else step(True, stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        g_att.replay() if g_att else step(False, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    att_us = e0.elapsed_time(e1) * 1e3 / args.steps
    flops = extend_flops(w)
    achieved = flops / (att_us * 1e-6) / 1e12
    print(f"[bench] {mode}: extend attention {att_us:.1f} us ({achieved:.1f} TFLOP/s), step {ms_per_step * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = extend_cpu_baseline(w)
    line = {
        "metric": EXTEND_METRIC.replace("ISO3", w.fmt_k.upper()), "value": round(ms_per_step * 1e3, 3),
        "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": f"f16/bf16 mfma, {w.fmt_k} cells",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "prefix": P, "n_new": N, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "k_format": w.fmt_k, "v_format": w.fmt_v,
                   "step": "extend attention over the packed prefix + causal new tokens, then pack the new tokens",
                   "launch": mode},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "extend launch (k_extend_stage + k_extend_attn)", "launch_us": round(att_us, 3),
                     "algorithmic_flops": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def time_batches(stream, n_batches, per_batch, graph, eager):
    """Per-launch µs of each of n_batches batches of per_batch launches (a graph replay, or the eager
    launches), from HIP events recorded on the launch stream around each batch."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_batches)]
    for e0, e1 in evs:
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            eager()
        e1.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 / per_batch for a, b in evs]


def copy_probe(nbytes: int):
    """A plain copy of a known number of bytes (torch's elementwise copy kernel), five times: the
    per-dispatch FETCH_SIZE / WRITE_SIZE counters of this kernel calibrate those of the others."""
    import torch
    n = nbytes // 16 * 16
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 5}))


def read_probe(nbytes: int):
    """Context for the HBM roofline: the rate of a plain streaming read (torch's sum over a float32
    tensor of nbytes, which reads it once) and of a plain copy, timed with HIP events."""
    import torch
    n = nbytes // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    res = {}
    for name, fn, moved in (("read", lambda: x.sum(), nbytes), ("copy", lambda: y.copy_(x), 2 * nbytes)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        res[name] = {"us": round(us, 2), "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
    print(json.dumps({"probe_bytes": nbytes, **res}))


def page_probe(args):
    """The int8 decode kernel's page stream without its arithmetic (libkvq_probe.so): for each
    (waves, pages per wave, pages in flight, with / without scale loads) of a sweep, the per-launch µs
    and GB/s over the workload's cache shape, on cache copies that together exceed the MALL.  One
    JSON line per configuration."""
    import ctypes
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    lib = ctypes.CDLL(os.path.join(os.path.dirname(kvq.__file__), "libkvq_probe.so"))
    lib.kvq_probe_page_stream.restype = ctypes.c_int
    lib.kvq_probe_page_stream.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int32] * 8 + [ctypes.c_void_p] * 2
    lib.kvq_probe_sink_words.restype = ctypes.c_int
    lib.kvq_probe_sink_words.argtypes = [ctypes.c_int32] * 4
    w = make_workload(args.workload, args.ctx)
    if (w.fmt_k, w.fmt_v) != ("int8", "int8") or w.batch != 1:
        raise SystemExit("--page-probe takes a single-sequence int8 K + V workload")
    D, hkv, npg = w.head_dim, w.n_kv_heads, w.num_pages
    max_pages = int((w.seq_lens[0] + w.page_size - 1) // w.page_size)
    code_bytes, scale_halves = npg * hkv * 16 * D, npg * hkv * 16 * (D // 64)
    per_copy = 2 * code_bytes + 4 * scale_halves
    R = args.replicas or max(2, int(np.ceil(3 * MALL_BYTES / per_copy)) + 1)
    gen = torch.Generator(device="cuda").manual_seed(7)
    copies = []
    for _ in range(R):
        k = torch.randint(0, 256, (code_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
        v = torch.randint(0, 256, (code_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
        ks = torch.randint(0, 1 << 15, (scale_halves,), dtype=torch.int16, device="cuda", generator=gen)
        vs = torch.randint(0, 1 << 15, (scale_halves,), dtype=torch.int16, device="cuda", generator=gen)
        copies.append((k, v, ks, vs))
    table = torch.from_numpy(np.ascontiguousarray(w.block_table[0][:max_pages], dtype=np.int32)).cuda()
    stream = torch.cuda.current_stream()
    full = max_pages * hkv * (2 * 16 * D + 2 * 16 * (D // 64) * 2)     # codes and scales of every page
    sweep = [(4, 16, 2), (4, 16, 1), (4, 16, 3), (4, 8, 1), (4, 8, 2), (8, 8, 1), (8, 8, 2), (8, 4, 1),
             (4, 4, 2), (2, 16, 2), (8, 16, 2)]
    for waves, ppw, depth in sweep:
        for no_scales in (0, 1):
            n_sink = lib.kvq_probe_sink_words(max_pages, hkv, waves, ppw)
            sink = torch.empty(n_sink, dtype=torch.int32, device="cuda")

            def launch(r, st):
                k, v, ks, vs = copies[r]
                rc = lib.kvq_probe_page_stream(k.data_ptr(), v.data_ptr(), ks.data_ptr(), vs.data_ptr(),
                                               table.data_ptr(), max_pages, npg, hkv, D, waves, ppw, depth,
                                               no_scales, sink.data_ptr(), st.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"page probe failed ({rc})")

            for r in range(R):
                launch(r, stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(R):
                    launch(r, torch.cuda.current_stream())
            g.replay()
            torch.cuda.synchronize()
            us = time_batches(stream, 50, R, g, None)
            moved = full if not no_scales else max_pages * hkv * 2 * 16 * D
            med = float(np.median(us))
            print(json.dumps({"page_probe": w.name, "waves": waves, "pages_per_wave": ppw, "in_flight": depth,
                              "scales": not no_scales, "workgroups": n_sink // waves, "cache_replicas": R,
                              "us_p50": round(med, 3), "us_p10": round(float(np.percentile(us, 10)), 3),
                              "bytes": moved, "GB/s": round(moved / (med * 1e-6) / 1e9, 1)}), flush=True)
            del g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="moe_int8_decode",
                    help="moe_int8_decode (default), moe_int8_decode_64k, tiny_int8_decode, batched_int8_decode, k8v4_verify, "
                         "iso3_extend, "
                         "int8_extend, moe_q4h_decode, moe_iso3_decode, batched_iso3_decode, moe_iso4_decode, "
                         "moe_k8v32_decode, moe_k32v8_decode")
    ap.add_argument("--ctx", type=int, default=0,
                    help="context length for the single-sequence moe_* decode workloads (default: their own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--unfused", action="store_true",
                    help="run quantize-on-write and decode as separate launches even where they can be fused")
    ap.add_argument("--replicas", type=int, default=0, help="cache copies to rotate (0 = enough to exceed the MALL)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run only a plain device copy of BYTES (calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="BYTES",
                    help="time only a plain streaming read and a plain copy of BYTES (context for the roofline)")
    ap.add_argument("--page-probe", action="store_true",
                    help="time only the int8 decode kernel's page stream (no arithmetic) over a sweep of launch "
                         "shapes, with and without the scale loads, on the workload's cache shape")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the hot path runs on one GPU "
              f"per process, with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_paged_kv_kvq_amd as kvq
    from synth import dev_bf16, dev_i32, token_lists

    torch.cuda.set_device(0)
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.read_probe:
        return read_probe(args.read_probe)
    kvq.lib()
    if args.page_probe:
        return page_probe(args)
    if args.workload in ("iso3_extend", "int8_extend"):
        return bench_extend(args)
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = make_workload(args.workload, args.ctx)
    cb_k, ns_k = kvq.cell_bytes(w.fmt_k, w.head_dim)
    cb_v, ns_v = kvq.cell_bytes(w.fmt_v, w.head_dim)
    cache_bytes = w.num_pages * w.n_kv_heads * 16 * ((cb_k + 2 * ns_k) + (cb_v + 2 * ns_v))
    # enough copies to exceed three times the Infinity Cache (capped: a tiny cache stays latency-bound)
    R = args.replicas or min(64, max(2, int(np.ceil(3 * MALL_BYTES / cache_bytes)) + 1))

    pre = token_lists(w, "prefix")
    step = token_lists(w, "step")
    block_table = dev_i32(w.block_table)
    seq_lens = dev_i32(w.seq_lens)
    pages = kvq.Pages(block_table, seq_lens)
    caches = []
    fill_us = []
    if pre is not None:
        p_seq, p_pos, p_k, p_v = dev_i32(pre[0]), dev_i32(pre[1]), dev_bf16(pre[2]), dev_bf16(pre[3])
    for r in range(R):
        c = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
        if pre is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            kvq.kvq_append(c, pages, p_k, p_v, p_seq, p_pos)
            e1.record()
            e1.synchronize()
            fill_us.append(e0.elapsed_time(e1) * 1e3)
        caches.append(c)
    if fill_us:
        # the cache fill (outside the timed steps): one multi-token append of every prefix token
        n_fill = len(pre[0])
        fill_bytes = n_fill * w.n_kv_heads * (2 * 2 * w.head_dim + (cb_k + 2 * ns_k) + (cb_v + 2 * ns_v))
        f_med = float(np.median(fill_us))
        print(f"[bench] cache fill: kvq_append of {n_fill} tokens, median {f_med:.1f} us over {len(fill_us)} fills, "
              f"{fill_bytes / f_med / 1e3:.0f} GB/s (bf16 read + cells written)", file=sys.stderr, flush=True)
        del p_seq, p_pos, p_k, p_v
    s_seq, s_pos, s_k, s_v = (dev_i32(step[0]), dev_i32(step[1]), dev_bf16(step[2]), dev_bf16(step[3]))
    # the fused call takes the step's tokens as [batch][n_q][n_kv_heads][head_dim] (sequence, then position)
    f_k = s_k.view(w.batch, w.n_step, w.n_kv_heads, w.head_dim) if fusable(w) else None
    f_v = s_v.view(w.batch, w.n_step, w.n_kv_heads, w.head_dim) if fusable(w) else None
    q = dev_bf16(w.q)
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = torch.empty((w.batch, w.n_q, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ws_bytes = kvq.kvq_decode_workspace_bytes(caches[0], w.batch, w.max_pages, w.n_q, w.n_q_heads)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {R} cache replicas of {cache_bytes / 1e6:.1f} MB; warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    # int8 K and V: the step is one fused launch sequence (the step's cells are encoded inside the
    # decode kernel); otherwise quantize-on-write, then decode.  The step's tokens are ordered by
    # sequence, then position, which is the fused call's [batch][n_q] order.
    fused = fusable(w) and not args.unfused

    def one_step(i, stream):
        c = caches[i % R]
        if fused:
            kvq.kvq_decode_attn_append(c, pages, f_k, f_v, q, q_lens=q_lens, sm_scale=w.sm_scale, out=out,
                                       workspace=ws, stream=stream)
            return
        kvq.kvq_append(c, pages, s_k, s_v, s_seq, s_pos, stream=stream)
        kvq.kvq_decode_attn(c, pages, q, q_lens=q_lens, sm_scale=w.sm_scale, out=out, workspace=ws, stream=stream)

    def decode_one(i, stream):
        if fused:
            kvq.kvq_decode_attn_append(caches[i], pages, f_k, f_v, q, q_lens=q_lens, sm_scale=w.sm_scale,
                                       out=out, workspace=ws, stream=stream)
        else:
            kvq.kvq_decode_attn(caches[i], pages, q, q_lens=q_lens, sm_scale=w.sm_scale, out=out,
                                workspace=ws, stream=stream)

    def decode_batch(stream):
        for i in range(R):
            decode_one(i, stream)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        one_step(i, stream)
    torch.cuda.synchronize()

    # The launches of a step are captured in HIP graphs (one per cache copy) and replayed, so the
    # timed loop measures the GPU rather than the Python launch path; eager launches if capture fails.
    # Steps are captured R to a graph, one per cache copy in order (as a model's decode graph holds
    # its layers' attention launches back to back, with no host round trip between them), plus one
    # graph per single step for a remainder of the K timed steps.
    graphs, round_graph, dec_graph, mode = None, None, None, "eager"
    if not args.no_graph:
        try:
            graphs = []
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    one_step(r, torch.cuda.current_stream())
                graphs.append(g)
            round_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(round_graph):
                for r in range(R):
                    one_step(r, torch.cuda.current_stream())
            dec_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(dec_graph):
                decode_batch(torch.cuda.current_stream())
            for g in graphs:
                g.replay()
            round_graph.replay()
            dec_graph.replay()
            torch.cuda.synchronize()
            mode = "hip-graph"
        except Exception as e:  # noqa: BLE001
            print(f"[bench] graph capture unavailable ({e}); timing eager launches", file=sys.stderr, flush=True)
            graphs, round_graph, dec_graph = None, None, None
    stream = torch.cuda.current_stream()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for _ in range(args.steps // R):
            round_graph.replay()
        for i in range(args.steps % R):
            graphs[i].replay()
    else:
        for i in range(args.steps):
            one_step(i, stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # Roofline of the decode attention launch: HIP events on the launch stream around batches of
    # back-to-back decode launches, one per cache copy in turn (so each reads HBM, not cache), so
    # the events' own fixed cost is spread over the batch.  At least 20 batches whatever --steps is.
    # At least 100 batches whatever --steps is (a few milliseconds of GPU time): their spread gives the
    # percentiles.  (Events around single one-launch graph replays would add each replay's own launch
    # cost, about 7 us here, to every sample.)
    n_batches, per_batch = max(100, args.steps // R), R
    dec_us = time_batches(stream, n_batches, per_batch, dec_graph, lambda: decode_batch(stream))
    dec_avg = float(np.mean(dec_us))
    algo = algorithmic_bytes(w, cb_k, ns_k, cb_v, ns_v, fused)
    achieved = algo / (dec_avg * 1e-6) / 1e9
    # Warm: the same launches all on one cache copy, which then stays in the 256 MB Infinity Cache
    # (when it fits): context for the MALL-defeated figures above, not a headline.
    warm_us = None
    if R > 1:
        warm_graph = None
        if graphs:
            warm_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(warm_graph):
                for _ in range(R):
                    decode_one(0, torch.cuda.current_stream())
            warm_graph.replay()
            torch.cuda.synchronize()
        warm_us = float(np.mean(time_batches(stream, 20, R, warm_graph,
                                             lambda: [decode_one(0, stream) for _ in range(R)])))
    pct = {k: round(float(np.percentile(dec_us, q)), 3) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    # The dominant kernel alone: the same algorithmic bytes over the split kernel's cold median from
    # the committed rocprofv3 trace of the current kernel source (None when the source has changed since)
    rk = recorded_kernel(w.name) if fused else None
    kernel_level = None if rk is None else {
        "kernel": rk["kernel"], "median_us": rk["median_us"],
        "achieved": round(algo / (rk["median_us"] * 1e-6) / 1e9, 1),
        "frac": round(algo / (rk["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": "rocprofv3 kernel trace, committed profile (cold-phase median)"}
    print(f"[bench] {mode}: decode launch avg {dec_avg:.2f} us over {n_batches} x {per_batch} launches "
          f"(p10/p50/p90 {pct['p10']}/{pct['p50']}/{pct['p90']}), step {ms_per_step * 1e3:.2f} us, "
          f"{achieved:.0f} GB/s; warm {warm_us if warm_us is None else round(warm_us, 2)} us",
          file=sys.stderr, flush=True)

    cpu = parity = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample; parity of the benched step", file=sys.stderr,
              flush=True)
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline(w, gpu_out=out.cpu().numpy(), gpu_cache=caches[0])

    line = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "/".join(dict.fromkeys({"int8": "int8", "q4h": "q4", "iso3": "iso3", "iso4": "iso4", "f32": "f32"}[f]
                                          for f in (w.fmt_k, w.fmt_v))),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": int(w.seq_lens.max()), "n_q": w.n_q,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "k_format": w.fmt_k, "v_format": w.fmt_v,
                   "step": ("quantize-on-write of the new K/V token(s) fused into decode attention" if fused
                            else "append new K/V token(s), then decode attention"), "cache_replicas": R,
                   "launch": mode, "steps_per_graph": R if graphs else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(w.name),
                     "kernel": ("fused quantize-on-write + decode attention launch (split-K kernel encoding "
                                "the step's cells + log-sum-exp combine kernel)" if fused else
                                "decode attention launch (split-K kernel + log-sum-exp combine kernel)"),
                     "launch_us": round(dec_avg, 3), "algorithmic_bytes": int(algo),
                     "kernel_level": kernel_level,
                     "timing": f"HIP events around {n_batches} batches of {per_batch} back-to-back launches, "
                               f"one per cache copy"},
        "launch_us_percentiles": {**pct, "n": n_batches,
                                  "what": f"per-launch mean of each batch of {per_batch} back-to-back launches"},
        "warm": None if warm_us is None else {
            "launch_us": round(warm_us, 3), "GB/s": round(algo / (warm_us * 1e-6) / 1e9, 1),
            "what": "the same launches on one cache copy (resident in the 256 MB Infinity Cache when it fits)"},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
