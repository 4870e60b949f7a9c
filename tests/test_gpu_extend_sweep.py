"""GPU parity over a seeded sweep of extend (prefill chunk) configurations, for ISO3 and int8 prefixes.

Each case draws a batch of 1-4 sequences with ragged prefix lengths (empty, single-cell, tile-edge
and longer prefixes) and ragged chunks (empty chunks included), a grouping of query heads onto KV
heads (1 to 32 per KV head, sometimes through an explicit uneven head map), and runs kvq_extend_attn
with deferred packing: the attention must meet the oracle (max-abs 1e-3, cosine > 0.9999 over the
tensor and every row) and the slabs after packing must hold the oracle's encoding of every token,
byte for byte.
"""
import numpy as np
import pytest

import synth
from kvq_testutil import assert_attention_close, assert_slabs_equal, oracle_stores
from test_gpu_extend import oracle_extend, run_extend

HEADS = [(8, 2), (4, 4), (16, 1), (32, 1), (32, 8), (12, 4), (6, 3)]
CASES_PER_FMT = 24
COST_BUDGET = 1_500_000    # sum over sequences of chunk x (prefix + chunk), times the query heads


def _lengths(rng, batch):
    pre, new = [], []
    for _ in range(batch):
        u = rng.random()
        pre.append(0 if u < 0.15 else int(rng.choice([1, 16, 63, 64, 65, 128])) if u < 0.4
                   else int(rng.integers(2, 1500)))
        v = rng.random()
        new.append(0 if v < 0.1 else int(rng.choice([1, 31, 32, 33, 64])) if v < 0.4 else int(rng.integers(2, 200)))
    return pre, new


def _case(fi, k):
    fmt = ("iso3", "int8")[fi]
    rng = np.random.default_rng(5000 + 100 * fi + k)
    for _ in range(200):
        hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
        head_map = None
        if hkv > 1 and rng.random() < 0.3:
            # uneven: the last KV head idle, at most 32 query heads on one KV head
            head_map = [int(h % (hkv - 1)) for h in range(hq)]
            if max(np.bincount(head_map)) > 32:
                continue
        pre, new = _lengths(rng, int(rng.integers(1, 5)))
        if sum(new) == 0:
            new[0] = int(rng.integers(1, 40))
        cost = sum(n * (p + n) for p, n in zip(pre, new)) * hq
        if cost > COST_BUDGET:
            continue
        return dict(fmt=fmt, pre=pre, new=new, hq=hq, hkv=hkv, head_map=head_map, seed=6000 + 100 * fi + k)
    raise AssertionError("no case within the limits")


CASES = [(fi, k) for fi in range(2) for k in range(CASES_PER_FMT)]


@pytest.mark.gpu
@pytest.mark.parametrize("fi,k", CASES, ids=[f"{('iso3', 'int8')[f]}-{k}" for f, k in CASES])
def test_extend_sweep(fi, k):
    c = _case(fi, k)
    w = synth.ragged_extend(c["pre"], c["new"], seed=c["seed"], n_q_heads=c["hq"], n_kv_heads=c["hkv"],
                            fmt=c["fmt"])
    print(f"[extend sweep] {c['fmt']} Hq={c['hq']} Hkv={c['hkv']} map={c['head_map']} prefix={c['pre']} "
          f"new={c['new']}", flush=True)
    cache, got = run_extend(w, head_map=c["head_map"])
    ref = oracle_extend(w, head_map=c["head_map"])
    m = assert_attention_close(got, ref)
    sk, sv = oracle_stores(w)
    assert_slabs_equal(cache, sk, sv)
    print(f"[extend sweep] max-abs {m[0]:.2e} cosine {m[1]:.8f} min row cosine {m[2]:.8f}", flush=True)


def test_extend_sweep_cases_within_limits():
    """The sweep's cases are drawn as described (runs without a GPU)."""
    for fi, k in CASES:
        c = _case(fi, k)
        assert 1 <= len(c["pre"]) <= 4 and sum(c["new"]) > 0
        g = max(np.bincount(c["head_map"])) if c["head_map"] else c["hq"] // c["hkv"]
        assert g <= 32
