"""CPU tests of the Python binding's argument checks: every tensor whose size the kernels trust is
compared with the cache and page-table descriptors (shape, dtype, device) and a mismatch raises
before the library is called.  The cache lives in host memory here, so a call that passed every
shape check would still stop at the last check (the slabs must be on a GPU): no kernel is launched.
"""
import pytest
import torch

from quantized_paged_kv_kvq_amd import kvq

B, NQ, HQ, HKV, D, MP = 2, 3, 8, 2, 128, 4


@pytest.fixture
def cp():
    cache = kvq.PagedKVCache(16, HKV, D, "int8", "int8", device="cpu")
    pages = kvq.Pages(torch.zeros((B, MP), dtype=torch.int32), torch.full((B,), 40, dtype=torch.int32))
    return cache, pages


def q_(b=B, nq=NQ, hq=HQ, d=D, dtype=torch.bfloat16):
    return torch.zeros((b, nq, hq, d), dtype=dtype)


def kv_(b=B, nq=NQ, h=HKV, d=D):
    return torch.zeros((b, nq, h, d), dtype=torch.bfloat16)


def test_pages_seq_lens_one_per_sequence():
    with pytest.raises(ValueError, match="seq_lens"):
        kvq.Pages(torch.zeros((B, MP), dtype=torch.int32), torch.zeros((B + 1,), dtype=torch.int32))


@pytest.mark.parametrize("bad,match", [
    (dict(b=B + 1), "q must have shape"),             # batch differs from the page table
    (dict(d=D // 2), "q must have shape"),            # head_dim differs from the cache
    (dict(dtype=torch.float16), "q must be"),
])
def test_decode_q_shape(cp, bad, match):
    cache, pages = cp
    with pytest.raises((ValueError, TypeError), match=match):
        kvq.kvq_decode_attn(cache, pages, q_(**bad))


def test_decode_q_lens_out_head_map(cp):
    cache, pages = cp
    with pytest.raises(ValueError, match="q_lens"):
        kvq.kvq_decode_attn(cache, pages, q_(), q_lens=torch.zeros(B * NQ - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        kvq.kvq_decode_attn(cache, pages, q_(), out=torch.zeros((B, NQ, HQ, D - 1), dtype=torch.float32))
    with pytest.raises(TypeError, match="out"):
        kvq.kvq_decode_attn(cache, pages, q_(), out=torch.zeros((B, NQ, HQ, D), dtype=torch.float16))
    with pytest.raises(ValueError, match="head_map"):
        kvq.kvq_decode_attn(cache, pages, q_(), head_map=[0] * (HQ - 1))


def test_fused_decode_new_tokens(cp):
    cache, pages = cp
    with pytest.raises(ValueError, match="k_new"):
        kvq.kvq_decode_attn_append(cache, pages, kv_(nq=NQ - 1), kv_(), q_())
    with pytest.raises(ValueError, match="v_new"):
        kvq.kvq_decode_attn_append(cache, pages, kv_(), kv_(h=HKV + 1), q_())


def test_correct_shapes_still_need_a_gpu(cp):
    cache, pages = cp
    with pytest.raises(ValueError, match="on a GPU"):
        kvq.kvq_decode_attn(cache, pages, q_())
    with pytest.raises(ValueError, match="on a GPU"):
        kvq.kvq_decode_attn_append(cache, pages, kv_(), kv_(), q_())


def test_append_token_arrays(cp):
    cache, pages = cp
    seq, pos = torch.zeros(5, dtype=torch.int32), torch.zeros(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="k_new"):
        kvq.kvq_append(cache, pages, torch.zeros((5, HKV, D + 64), dtype=torch.bfloat16), None, seq, pos)
    with pytest.raises(ValueError, match="tok_pos"):
        kvq.kvq_append(cache, pages, torch.zeros((5, HKV, D), dtype=torch.bfloat16), None, seq,
                       torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="on a GPU"):
        kvq.kvq_append(cache, pages, torch.zeros((5, HKV, D), dtype=torch.bfloat16), None, seq, pos)


def test_extend_shapes(cp):
    cache, pages = cp
    n = 10
    q = torch.zeros((n, HQ, D), dtype=torch.bfloat16)
    kn = torch.zeros((n, HKV, D), dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, n], dtype=torch.int32)
    with pytest.raises(ValueError, match="k_new"):
        kvq.kvq_extend_attn(cache, pages, q, kn[:-1], kn, cu, 6)
    with pytest.raises(ValueError, match="cu_new"):
        kvq.kvq_extend_attn(cache, pages, q, kn, kn, cu[:-1], 6)
    with pytest.raises(ValueError, match="out"):
        kvq.kvq_extend_attn(cache, pages, q, kn, kn, cu, 6, out=torch.zeros((n, HQ + 1, D)))
    with pytest.raises(ValueError, match="on a GPU"):
        kvq.kvq_extend_attn(cache, pages, q, kn, kn, cu, 6)


def test_gather_out_shape(cp):
    cache, pages = cp
    with pytest.raises(ValueError, match="out"):
        kvq.kvq_dequant_gather(cache, pages, "k", 0, 0, 7, out=torch.zeros((8, HKV, D)))
    with pytest.raises(ValueError, match="on a GPU"):
        kvq.kvq_dequant_gather(cache, pages, "k", 0, 0, 7)
