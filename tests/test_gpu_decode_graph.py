"""GPU parity of decode with sequences that leave whole context splits empty, and of append + decode
(every store format mix the decode supports) and extend (ISO3 and int8 prefixes) captured in a HIP
graph: the graph is replayed several times, with eager work between the replays, and every replay
must reproduce the eager result exactly.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, dev_bf16, dev_i32, gpu_append, gpu_cache, oracle_decode,
                          oracle_stores)

pytestmark = pytest.mark.gpu


def _decode(w):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn(cache, pages, dev_bf16(w.q), q_lens=q_lens, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_decode_empty_splits_match_oracle():
    """Lengths 5000, 1, 0 and 2048 in one batch: most splits of the short sequences see no cell."""
    w = synth.ragged_decode("int8", "int8", [5000, 1, 0, 2048], seed=41, n_q_heads=16, n_kv_heads=2, head_dim=256)
    sk, sv = oracle_stores(w)
    assert_attention_close(_decode(w), oracle_decode(w, sk, sv))


def test_verify_k8v4_ragged_windows():
    w = synth.ragged_decode("int8", "q4h", [3000, 77], seed=42, n_q=3, n_q_heads=16, n_kv_heads=2, head_dim=256,
                            q_len_back=[2, 1, 0])
    sk, sv = oracle_stores(w)
    assert_attention_close(_decode(w), oracle_decode(w, sk, sv))


@pytest.mark.parametrize("fk,fv", [("int8", "int8"), ("int8", "f32"), ("f32", "int8"), ("iso4", "iso4"),
                                   ("q4h", "q4h"), ("iso3", "iso3")])
def test_decode_graph_replays(fk, fv):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_decode(fk, fv, [4096, 300], seed=43, n_q_heads=16, n_kv_heads=2, head_dim=256)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    step = [x for x in __import__("kvq_testutil").token_lists(w, "step")]
    s_seq, s_pos, s_k, s_v = dev_i32(step[0]), dev_i32(step[1]), dev_bf16(step[2]), dev_bf16(step[3])
    q = dev_bf16(w.q)
    out = torch.empty((w.batch, w.n_q, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nbytes = kvq.kvq_decode_workspace_bytes(cache, pages.batch, pages.max_pages, w.n_q, w.n_q_heads)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step_fn():
        kvq.kvq_append(cache, pages, s_k, s_v, s_seq, s_pos)
        kvq.kvq_decode_attn(cache, pages, q, sm_scale=w.sm_scale, out=out, workspace=ws)

    step_fn()
    torch.cuda.synchronize()
    eager = out.clone()
    sk, sv = oracle_stores(w)
    assert_attention_close(eager.cpu().numpy(), oracle_decode(w, sk, sv))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step_fn()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn()
    for i in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager.cpu().numpy()), f"replay {i} differs from the eager run"
        del junk


@pytest.mark.parametrize("fmt", ["int8", "iso3"])
def test_extend_graph_replays(fmt):
    """Extend (stage + attention + deferred packing) captured once and replayed with eager work between
    the replays: every replay reproduces the eager output."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_extend([300, 70], [100, 45], seed=44, fmt=fmt)
    pre, new = w.prefix_lens(), w.new_lens()
    cache = kvq.PagedKVCache(w.num_pages, w.n_kv_heads, w.head_dim, w.fmt_k, w.fmt_v, quat=w.quat)
    pages = kvq.Pages(dev_i32(w.block_table), dev_i32(pre))
    tok_seq = np.concatenate([np.full(int(pre[b]), b, np.int32) for b in range(w.batch)])
    tok_pos = np.concatenate([np.arange(int(pre[b]), dtype=np.int32) for b in range(w.batch)])
    kvq.kvq_append(cache, pages, dev_bf16(np.concatenate([w.k[b][:int(pre[b])] for b in range(w.batch)])),
                   dev_bf16(np.concatenate([w.v[b][:int(pre[b])] for b in range(w.batch)])), dev_i32(tok_seq),
                   dev_i32(tok_pos))
    kn = dev_bf16(np.concatenate([w.k[b][int(pre[b]):] for b in range(w.batch)]))
    vn = dev_bf16(np.concatenate([w.v[b][int(pre[b]):] for b in range(w.batch)]))
    cu = dev_i32(np.concatenate([[0], np.cumsum(new)]).astype(np.int32))
    q = dev_bf16(w.q)
    out = torch.empty((int(new.sum()), w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    nbytes = kvq.kvq_extend_workspace_bytes(cache, pages.batch, pages.max_pages, int(new.sum()), int(new.max()),
                                            w.n_q_heads)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step_fn():
        kvq.kvq_extend_attn(cache, pages, q, kn, vn, cu, int(new.max()), sm_scale=w.sm_scale, out=out,
                            pack_after=True, workspace=ws)

    step_fn()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step_fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn()
    for i in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager.cpu().numpy()), f"replay {i} differs from the eager run"
        del junk


def _prepared(w):
    """A filled cache, its pages and the device query of a decode workload."""
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    return cache, pages, dev_bf16(w.q), q_lens


def test_decode_workspace_reused_across_different_inputs():
    """One workspace for consecutive launches over different caches and queries (single-sequence
    decode and verify shapes, and a batch): the combine must read the partials of its own launch.
    Launches with the same inputs write the same partials, so only alternating inputs can show a
    stale read: every launch, eager and inside one replayed graph, must equal its own
    fresh-workspace result bit for bit."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    ws_ = [synth.moe_int8_decode(ctx=20000, seed=91), synth.k8v4_verify(ctx=9000, seed=92),
           synth.moe_int8_decode(ctx=20000, seed=93),
           synth.ragged_decode("int8", "int8", [3000, 700, 5000], seed=94, n_q_heads=16, n_kv_heads=2, head_dim=256),
           synth.k8v4_verify(ctx=100000, seed=95)]
    prep = [_prepared(w) for w in ws_]
    refs = [kvq.kvq_decode_attn(c, p, q, q_lens=ql, sm_scale=w.sm_scale) for w, (c, p, q, ql) in zip(ws_, prep)]
    torch.cuda.synchronize()
    for w, r, (c, p, q, ql) in list(zip(ws_, refs, prep))[:4]:    # and the fresh results are right
        sk, sv = oracle_stores(w)
        assert_attention_close(r.cpu().numpy(), oracle_decode(w, sk, sv))
    nbytes = max(kvq.kvq_decode_workspace_bytes(c, p.batch, p.max_pages, w.n_q, w.n_q_heads)
                 for w, (c, p, q, ql) in zip(ws_, prep))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(r) for r in refs]
    order = [0, 1, 4, 2, 3, 0, 4, 2, 1, 0, 3, 4, 2]

    def run_all():
        for i in order:
            w, (c, p, q, ql) = ws_[i], prep[i]
            kvq.kvq_decode_attn(c, p, q, q_lens=ql, sm_scale=w.sm_scale, out=outs[i], workspace=ws)

    for i in order:                                               # eager, checked after each launch
        w, (c, p, q, ql) = ws_[i], prep[i]
        kvq.kvq_decode_attn(c, p, q, q_lens=ql, sm_scale=w.sm_scale, out=outs[i], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], refs[i]), f"eager launch of workload {i}"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"replay {rep}, workload {i}"
