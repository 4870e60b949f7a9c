"""GPU test of kvq_decode_attn_noalloc (decode without a workspace: the split partials go to the
library's own per-GPU scratch), through the C ABI.  Each call's output must equal kvq_decode_attn's
on the same inputs bit for bit (same kernels, same launch plan) and the oracle's within the parity
bar.  Two calls in a row, the second with a smaller input, so the scratch holds the first call's
partials when the second runs; then other decode kernels (k8v4 verify, ISO3) through the scratch.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, dev_bf16, dev_i32, gpu_append, gpu_cache, oracle_decode,
                          oracle_stores)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_paged_kv_kvq_amd as kvq
    kvq.lib()


def both(w):
    """(noalloc output, workspace-path output) on one cache, as numpy."""
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q = dev_bf16(w.q)
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = torch.full((w.batch, w.n_q, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attn_noalloc(cache, pages, q, q_lens=q_lens, sm_scale=w.sm_scale, out=out)
    ref = kvq.kvq_decode_attn(cache, pages, q, q_lens=q_lens, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


def check(w):
    print(f"[noalloc] {w.name} {w.fmt_k}/{w.fmt_v} B={w.batch} lens={list(w.seq_lens)[:6]} n_q={w.n_q}", flush=True)
    got, ref = both(w)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "noalloc and workspace outputs differ"
    sk, sv = oracle_stores(w)
    assert_attention_close(got, oracle_decode(w, sk, sv))


def test_noalloc_two_calls_second_smaller():
    check(synth.ragged_decode("int8", "int8", [9000, 20000, 700], seed=81, n_q_heads=16, n_kv_heads=2, head_dim=256))
    check(synth.ragged_decode("int8", "int8", [300, 17], seed=82, n_q_heads=16, n_kv_heads=2, head_dim=256))


def test_noalloc_other_kernels():
    check(synth.k8v4_verify(ctx=5000, seed=83))
    check(synth.ragged_decode("iso3", "iso3", [2000, 33], seed=84, n_q_heads=8, n_kv_heads=2, head_dim=128))
    check(synth.ragged_decode("int8", "int8", [1], seed=85, n_q_heads=4, n_kv_heads=1, head_dim=128))


def test_noalloc_refuses_calls_beyond_its_scratch():
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    cache = kvq.PagedKVCache(64, 8, 128, "int8", "int8")
    pages = kvq.Pages(torch.zeros((64, 4096), dtype=torch.int32, device="cuda"),
                      torch.zeros(64, dtype=torch.int32, device="cuda"))
    q = torch.zeros((64, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KVQError, match="scratch"):
        kvq.kvq_decode_attn_noalloc(cache, pages, q)
