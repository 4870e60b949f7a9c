"""GPU parity of decode with sequences that leave whole context splits empty, and of append +
decode captured in a HIP graph: the graph is replayed several times, with eager work between the
replays, and every replay must reproduce the eager result exactly.
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


def test_decode_graph_replays():
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    w = synth.ragged_decode("int8", "int8", [4096, 300], seed=43, n_q_heads=16, n_kv_heads=2, head_dim=256)
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
