"""GPU parity over a seeded sweep of decode / verify configurations for every store mix.

Each case draws a batch of ragged lengths (empty sequences and page-edge lengths included), a
grouping of query heads onto KV heads (sometimes through an explicit, uneven head map), a head_dim
and a verify window of 1-3 query tokens with per-query causal lengths, within the row limits the
library states for the mix.  The launch plans then visit their launch shapes and split sizes
(64-, 32- and fewer-page splits, 4- and 8-wave workgroups, one split writing the output directly),
and every case must meet the oracle: codes, scales and norms byte for byte, attention within
max-abs 1e-3 and cosine > 0.9999 over the tensor and every row.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import (assert_attention_close, assert_slabs_equal, dev_bf16, dev_i32, gpu_append, gpu_cache,
                          oracle_decode, oracle_stores)

# (K format, V format, head_dims, largest n_q * query heads of one KV head)
MIXES = [
    ("int8", "int8", (64, 128, 256), 32),
    ("int8", "q4h", (256,), 32),
    ("q4h", "q4h", (256,), 16),
    ("iso3", "iso3", (128, 256), 16),
    ("iso4", "iso4", (128, 256), 16),
    ("int8", "f32", (128, 256), 32),
    ("f32", "int8", (128, 256), 32),
]
CASES_PER_MIX = 16
LONG_CASES = 2               # the last cases of a mix: one sequence of 20,000-60,000 tokens over 2 KV heads
HEADS = [(8, 2), (16, 2), (4, 4), (16, 1), (32, 8), (12, 4)]
CELL_BUDGET = 60000          # sum of lengths x KV heads per case: the oracle stays within seconds


def _lengths(rng, batch):
    out = []
    for _ in range(batch):
        u = rng.random()
        if u < 0.1:
            out.append(0)
        elif u < 0.25:
            out.append(int(rng.choice([1, 15, 16, 17, 1023, 1024, 1025])))
        elif u < 0.45:
            out.append(int(rng.integers(1, 64)))
        elif u < 0.85:
            out.append(int(rng.integers(100, 3000)))
        else:
            out.append(int(rng.integers(4000, 12000)))
    return out


def _case(mix_index, k):
    fk, fv, dims, max_rows = MIXES[mix_index]
    rng = np.random.default_rng(1000 * mix_index + k)
    D = int(rng.choice(dims))
    if k >= CASES_PER_MIX - LONG_CASES:
        n_q = int(rng.integers(1, 3))
        hq = 8 if n_q * 8 <= max_rows else 4
        return dict(fk=fk, fv=fv, D=D, hq=hq, hkv=2, n_q=n_q, lens=[int(rng.integers(20000, 60000))],
                    head_map=None, seed=7000 + 100 * mix_index + k)
    for _ in range(100):
        hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
        n_q = int(rng.integers(1, 4))
        head_map = None
        if rng.random() < 0.3 and hkv > 1:
            # an uneven map that leaves the last KV head idle: rows per KV head up to ceil(hq / (hkv - 1))
            head_map = [int(h % (hkv - 1)) for h in range(hq)]
            g = max(np.bincount(head_map, minlength=hkv))
        else:
            g = hq // hkv
        if n_q * g > max_rows:
            continue
        batch = int(rng.integers(1, 5))
        lens = _lengths(rng, batch)
        if max(lens) < n_q:                  # at least one sequence sees every query token's window
            lens[0] = n_q + int(rng.integers(0, 40))
        if sum(lens) * hkv > CELL_BUDGET:
            continue
        return dict(fk=fk, fv=fv, D=D, hq=hq, hkv=hkv, n_q=n_q, lens=lens, head_map=head_map,
                    seed=7000 + 100 * mix_index + k)
    raise AssertionError("no case within the limits")


CASES = [(m, k) for m in range(len(MIXES)) for k in range(CASES_PER_MIX)]


@pytest.mark.gpu
@pytest.mark.parametrize("mix,k", CASES, ids=[f"{MIXES[m][0]}-{MIXES[m][1]}-{k}" for m, k in CASES])
def test_decode_sweep(mix, k):
    import torch
    import quantized_paged_kv_kvq_amd as kvq
    c = _case(mix, k)
    back = list(range(c["n_q"] - 1, -1, -1)) if c["n_q"] > 1 else None
    w = synth.ragged_decode(c["fk"], c["fv"], c["lens"], seed=c["seed"], n_q=c["n_q"], q_len_back=back,
                            n_q_heads=c["hq"], n_kv_heads=c["hkv"], head_dim=c["D"])
    print(f"[sweep] {c['fk']}/{c['fv']} D={c['D']} Hq={c['hq']} Hkv={c['hkv']} n_q={c['n_q']} "
          f"map={c['head_map']} lens={c['lens']}", flush=True)
    cache, pages = gpu_cache(w)
    gpu_append(w, cache, pages, "prefix")
    gpu_append(w, cache, pages, "step")
    q_lens = dev_i32(w.q_lens) if w.q_lens is not None else None
    out = kvq.kvq_decode_attn(cache, pages, dev_bf16(w.q), q_lens=q_lens, head_map=c["head_map"],
                              sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    m = assert_attention_close(out.cpu().numpy(), oracle_decode(w, sk, sv, head_map=c["head_map"]))
    print(f"[sweep] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)


def test_sweep_cases_within_limits():
    """The sweep's cases are drawn as described (runs without a GPU)."""
    for m, k in CASES:
        c = _case(m, k)
        g = max(np.bincount(c["head_map"], minlength=c["hkv"])) if c["head_map"] else c["hq"] // c["hkv"]
        long = k >= CASES_PER_MIX - LONG_CASES
        assert c["n_q"] * g <= MIXES[m][3] and sum(c["lens"]) * c["hkv"] <= (120000 if long else CELL_BUDGET)
