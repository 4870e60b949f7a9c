"""Pins for the fp64 attention oracle and the paged addressing."""
import numpy as np
import torch

from oracle import attention, paged
from oracle.numerics import bf16_to_f32
import synth


def sdpa64(q, K, V, scale, causal=False):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        scale=scale, is_causal=causal)
    return out[0].numpy()


def test_attend_matches_torch_sdpa_float64():
    rng = np.random.default_rng(13)
    q, K, V = rng.standard_normal((5, 64)), rng.standard_normal((300, 64)), rng.standard_normal((300, 64))
    got = attention.attend(q, K, V, 0.125)
    assert np.allclose(got, sdpa64(q, K, V, 0.125), rtol=0, atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, 16))
    V = rng.standard_normal((7, 16))
    assert np.allclose(attention.attend(q, rng.standard_normal((1, 16)), V[:1], 1.0), V[:1])   # single key
    K = np.zeros((7, 16))
    assert np.allclose(attention.attend(q, K, V, 1.0), V.mean(0))                                # equal scores
    assert np.all(attention.attend_lengths(q, K, V, [0, 0, 0], 1.0) == 0)                        # empty context
    # large score offsets do not overflow (max subtraction)
    assert np.allclose(attention.attend(q, K + 1e3, V, 1.0), V.mean(0))


def test_lengths_mask_is_prefix_attention():
    rng = np.random.default_rng(15)
    q, K, V = rng.standard_normal((4, 32)), rng.standard_normal((50, 32)), rng.standard_normal((50, 32))
    lens = [50, 49, 1, 17]
    got = attention.attend_lengths(q, K, V, lens, 0.3, chunk=3)
    for r, L in enumerate(lens):
        assert np.allclose(got[r], attention.attend(q[r:r + 1], K[:L], V[:L], 0.3)[0], atol=1e-13)


def test_split_lse_combine_equals_unsplit():
    # The identity the kernels' split-K path relies on, checked on the oracle's own definition.
    rng = np.random.default_rng(16)
    q, K, V = rng.standard_normal((2, 32)), rng.standard_normal((97, 32)), rng.standard_normal((97, 32))
    full = attention.attend(q, K, V, 0.2)
    cuts = [0, 10, 11, 60, 97]
    ms, ls, os_ = [], [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = 0.2 * q @ K[a:b].T
        m = s.max(1, keepdims=True)
        w = np.exp(s - m)
        ms.append(m), ls.append(w.sum(1, keepdims=True)), os_.append(w @ V[a:b])
    M = np.max(np.concatenate(ms, 1), 1, keepdims=True)
    num = sum(np.exp(m - M) * o for m, o in zip(ms, os_))
    den = sum(np.exp(m - M) * l for m, l in zip(ms, ls))
    assert np.allclose(num / den, full, atol=1e-13)


def _fill(w, fmt_k, fmt_v):
    sk = paged.Store.empty(fmt_k, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    sv = paged.Store.empty(fmt_v, w.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        pos = np.arange(L)
        paged.append(sk, w.block_table, np.full(L, b), pos, w.k[b], w.page_size, quat=w.quat)
        paged.append(sv, w.block_table, np.full(L, b), pos, w.v[b], w.page_size, quat=w.quat)
    return sk, sv


def test_locate_worked_example():
    """Paged addressing on a hand-worked table (strata PR #120, Tests: append and gather through a
    non-identity page table): token j of sequence b sits in slot j mod 16 of the page that the table
    names for block j div 16.  The expected pairs are written out, not recomputed."""
    table = np.array([[7, 3, 9, 0], [2, 11, 5, 4]], np.int32)
    seq = [0, 0, 0, 0, 0, 1, 1, 1, 1]
    pos = [0, 15, 16, 31, 40, 0, 17, 47, 63]
    page, slot = paged.locate(table, seq, pos, 16)
    assert page.tolist() == [7, 7, 3, 3, 9, 2, 11, 5, 4]
    assert slot.tolist() == [0, 15, 0, 15, 8, 0, 1, 15, 15]


def test_append_writes_exactly_the_located_cell():
    """One appended token changes only its own cell: page 9, slot 8 for token 40 of sequence 0 in the
    table above, every KV head of it, and nothing else in the store."""
    table = np.array([[7, 3, 9, 0], [2, 11, 5, 4]], np.int32)
    for fmt in ("int8", "q4h"):
        st = paged.Store.empty(fmt, 12, 2, 16, 256)
        x = synth.normal_bf16(np.random.default_rng(5), (1, 2, 256))
        paged.append(st, table, [0], [40], x, 16)
        changed = np.argwhere(st.codes.reshape(12, 2, 16, -1).any(axis=3))
        assert changed.tolist() == [[9, 0, 8], [9, 1, 8]]
        assert np.argwhere(st.scales.view(np.uint16).any(axis=3)).tolist() == [[9, 0, 8], [9, 1, 8]]


def test_paged_gather_independent_of_page_table():
    for fmt in ("int8", "q4h", "iso3"):
        D = 256 if fmt == "q4h" else 128
        w = synth.ragged_decode(fmt, fmt, [37, 64, 5], head_dim=D, seed=17)
        sk, _ = _fill(w, fmt, fmt)
        assert sorted(set(w.block_table[0][:3]) | set(w.block_table[1][:4])) != list(range(7))
        for b in range(w.batch):
            L = int(w.seq_lens[b])
            codes, scales = paged.encode_cells(fmt, bf16_to_f32(w.k[b]), w.quat)
            c2, s2 = paged.gather_raw(sk, w.block_table, b, 0, L, w.page_size)
            assert np.array_equal(codes, c2) and np.array_equal(scales.view(np.uint16), s2.view(np.uint16))


def test_decode_gqa_and_verify_rows():
    w = synth.ragged_decode("int8", "int8", [40, 23], n_q=3, q_len_back=[2, 1, 0], seed=18,
                            n_q_heads=8, n_kv_heads=2, head_dim=128)
    sk, sv = _fill(w, "int8", "int8")
    out = attention.decode(sk, sv, w.block_table, w.seq_lens, w.q, w.page_size, w.sm_scale, q_lens=w.q_lens)
    qf = bf16_to_f32(w.q).astype(np.float64)
    for b in range(w.batch):
        K = paged.gather(sk, w.block_table, b, 0, int(w.seq_lens[b]), w.page_size).astype(np.float64)
        V = paged.gather(sv, w.block_table, b, 0, int(w.seq_lens[b]), w.page_size).astype(np.float64)
        for t in range(3):
            L = int(w.q_lens[b, t])
            for h in range(8):
                ref = sdpa64(qf[b, t, h][None], K[:L, h // 4], V[:L, h // 4], w.sm_scale)[0]
                assert np.allclose(out[b, t, h], ref, atol=1e-6)
    # an explicit head map equal to the default gives the same result; MHA is Hq == Hkv
    hm = attention.default_head_map(8, 2)
    assert list(hm) == [0, 0, 0, 0, 1, 1, 1, 1]
    out2 = attention.decode(sk, sv, w.block_table, w.seq_lens, w.q, w.page_size, w.sm_scale,
                            q_lens=w.q_lens, head_map=hm)
    assert np.array_equal(out, out2)
    assert list(attention.default_head_map(4, 4)) == [0, 1, 2, 3]


def test_q4h_value_side_is_rotated_back():
    w = synth.ragged_decode("int8", "q4h", [33], seed=19, n_q_heads=4, n_kv_heads=1, head_dim=256)
    sk, sv = _fill(w, "int8", "q4h")
    out = attention.decode(sk, sv, w.block_table, w.seq_lens, w.q, w.page_size, w.sm_scale)
    # attention in the rotated basis followed by H equals attention over rotated-back values
    K = paged.gather(sk, w.block_table, 0, 0, 33, 16).astype(np.float64)
    Vr = paged.gather(sv, w.block_table, 0, 0, 33, 16, rotated=True).astype(np.float64)
    qf = bf16_to_f32(w.q).astype(np.float64)
    for h in range(4):
        o_rot = attention.attend(qf[0, 0, h][None], K[:, 0], Vr[:, 0], w.sm_scale)
        from oracle.q4h import hadamard_f64
        assert np.allclose(hadamard_f64(o_rot)[0], out[0, 0, h], atol=1e-6)
    # and the stored values approximate the bf16 inputs
    Vo = paged.gather(sv, w.block_table, 0, 0, 33, 16, rotated=False)
    assert np.mean(np.abs(Vo - bf16_to_f32(w.v[0]))) < 0.15


def test_extend_empty_prefix_is_causal_attention():
    w = synth.iso3_extend(prefix=0, n_new=40, seed=20, n_q_heads=4, n_kv_heads=2, head_dim=128)
    sk = paged.Store.empty("iso3", w.num_pages, 2, 16, 128)
    sv = paged.Store.empty("iso3", w.num_pages, 2, 16, 128)
    cu = np.array([0, 40])
    out = attention.extend(sk, sv, w.block_table, np.array([0]), w.q, w.k[0], w.v[0], cu, 16, w.sm_scale, quat=w.quat)
    qf = bf16_to_f32(w.q).astype(np.float64)
    kf = bf16_to_f32(w.k[0]).astype(np.float64)
    vf = bf16_to_f32(w.v[0]).astype(np.float64)
    for h in range(4):
        ref = sdpa64(qf[:, h], kf[:, h // 2], vf[:, h // 2], w.sm_scale, causal=True)
        assert np.allclose(out[:, h], ref, atol=1e-6)


def test_extend_with_prefix_and_row_sampling():
    w = synth.iso3_extend(prefix=50, n_new=20, seed=21, n_q_heads=4, n_kv_heads=2, head_dim=128, batch=2)
    sk = paged.Store.empty("iso3", w.num_pages, 2, 16, 128)
    sv = paged.Store.empty("iso3", w.num_pages, 2, 16, 128)
    for b in range(2):
        paged.append(sk, w.block_table, np.full(50, b), np.arange(50), w.k[b][:50], 16, quat=w.quat)
        paged.append(sv, w.block_table, np.full(50, b), np.arange(50), w.v[b][:50], 16, quat=w.quat)
    cu = np.array([0, 20, 40])
    kn = np.concatenate([w.k[0][50:], w.k[1][50:]])
    vn = np.concatenate([w.v[0][50:], w.v[1][50:]])
    out = attention.extend(sk, sv, w.block_table, np.array([50, 50]), w.q, kn, vn, cu, 16, w.sm_scale, quat=w.quat)
    qf = bf16_to_f32(w.q).astype(np.float64)
    for b in range(2):
        Kp = paged.gather(sk, w.block_table, b, 0, 50, 16, quat=w.quat).astype(np.float64)
        Vp = paged.gather(sv, w.block_table, b, 0, 50, 16, quat=w.quat).astype(np.float64)
        K = np.concatenate([Kp, bf16_to_f32(w.k[b][50:]).astype(np.float64)])
        V = np.concatenate([Vp, bf16_to_f32(w.v[b][50:]).astype(np.float64)])
        for i in (0, 7, 19):
            for h in range(4):
                ref = attention.attend(qf[20 * b + i, h][None], K[:51 + i, h // 2], V[:51 + i, h // 2], w.sm_scale)
                assert np.allclose(out[20 * b + i, h], ref[0], atol=1e-6)
    some = attention.extend(sk, sv, w.block_table, np.array([50, 50]), w.q, kn, vn, cu, 16, w.sm_scale,
                            quat=w.quat, rows=[3, 25])
    assert np.array_equal(some[[3, 25]], out[[3, 25]]) and np.all(some[[0, 30]] == 0)
