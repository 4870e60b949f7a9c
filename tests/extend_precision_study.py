"""Error budget of the ISO3 extend kernel's operand splits: a CPU study, not a test (pytest does not
collect it).

    python tests/extend_precision_study.py [random|peaked|two|sharp ...]

Emulates the extend kernel's arithmetic for one KV head -- prefix phase in the quaternion-rotated
basis (centroid levels S*c in fp16, the rotated and pre-scaled query in fp16 hi (+ lo), weights
p * n / S in fp16 hi (+ lo), products accumulated and rounded to binary32), chunk phase with bf16
operands (weights in bf16 hi (+ lo)) -- and reports the worst max-abs difference from fp64 attention
over the oracle's dequantised cells, for every combination of one or two parts per operand.
Inputs: seeded N(0,1) keys, values and queries, and three adversarial kinds: "peaked" (each query
matches one prefix key x2.5), "two" (two nearly equal matching keys), "sharp" (queries x4).
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from oracle import paged as opaged  # noqa: E402
from oracle import iso3 as oiso  # noqa: E402
import synth  # noqa: E402

S = 1.2495174
LOG2E = 1.4426950408889634


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def bf16(x):
    return synth.bf16_bits(np.asarray(x, np.float32)).astype(np.uint32) << 16


def bf16f(x):
    return (bf16(x)).view(np.float32)


def qmul(r, g):
    return oiso.quat_left_mul(r, g.reshape(*g.shape[:-1], -1, 4)).reshape(g.shape)


def split(x, kind, parts):
    x = np.asarray(x, np.float32)
    if kind == 'f16':
        hi = f16(x)
        lo = f16(x - hi)
    else:
        hi = (x.view(np.uint32) & np.uint32(0xffff0000)).view(np.float32)
        lo = bf16f(x - hi)
    return hi + lo if parts == 2 else hi


def emulate(P, q, kp_codes, kp_norm, vp_codes, vp_norm, kn, vn, quat, sm_scale, q_parts, w_parts, cw_parts):
    """q [R][D] f32 (bf16 values), rows r see P prefix keys + chunk keys 0..t_r (t_r given by row order)."""
    R, D = q.shape
    cs = oiso.centroids()
    lev = f16(S * cs)                                    # fp16 S*c
    Kf = lev[kp_codes].astype(np.float64)                # [P][D] rotated basis
    Vf = lev[vp_codes].astype(np.float64)
    qs = np.float32(np.float32(sm_scale) * np.float32(LOG2E)) / np.float32(S)
    qrot = qmul(quat, q.astype(np.float32)) * qs
    mx = np.max(np.abs(qrot), axis=1, keepdims=True)
    ex = 14 - np.frexp(mx)[1]
    x = np.ldexp(qrot, ex).astype(np.float32)
    qq = split(x, 'f16', q_parts).astype(np.float64)
    rs = np.ldexp(1.0, -ex).astype(np.float32)
    acc = (qq @ Kf.T).astype(np.float32)                 # [R][P] fp32 accumulate
    u = (acc * kp_norm[None, :].astype(np.float32)) * rs  # log2 units
    # chunk scores (bf16 exact operands)
    sl2 = np.float32(np.float32(sm_scale) * np.float32(LOG2E))
    uc = (q.astype(np.float64) @ kn.astype(np.float64).T).astype(np.float32) * sl2   # [R][N]
    N = kn.shape[0]
    out = np.zeros((R, D), np.float64)
    for r in range(R):
        t = r  # one query row per chunk token here
        sc = np.concatenate([u[r], uc[r, :t + 1]])
        m = np.max(sc)
        p = np.exp2((sc - m).astype(np.float32)).astype(np.float32)
        l = np.float32(np.sum(p[:P], dtype=np.float32) + np.sum(p[P:], dtype=np.float32))
        w = split(p[:P] * (vp_norm.astype(np.float32) / np.float32(S)), 'f16', w_parts).astype(np.float64)
        orot = (w @ Vf).astype(np.float32)
        o_pre = qmul(oiso.conjugate(quat), orot[None, :])[0].astype(np.float64)
        wc = split(p[P:], 'bf16', cw_parts).astype(np.float64)
        o_ch = wc @ vn[:t + 1].astype(np.float64)
        out[r] = (o_pre + o_ch) / l
    return out


def reference(P, q, Kd, Vd, kn, vn, sm_scale):
    R, D = q.shape
    out = np.zeros((R, D), np.float64)
    for r in range(R):
        K = np.concatenate([Kd, kn[:r + 1]]).astype(np.float64)
        V = np.concatenate([Vd, vn[:r + 1]]).astype(np.float64)
        s = sm_scale * (K @ q[r].astype(np.float64))
        w = np.exp(s - s.max())
        out[r] = w @ V / w.sum()
    return out


def case(P, N, seed, kind):
    rng = np.random.default_rng(seed)
    D = 128
    quat = synth.random_quaternion(seed + 7)
    K = rng.standard_normal((P + N, D)).astype(np.float32)
    V = rng.standard_normal((P + N, D)).astype(np.float32)
    q = rng.standard_normal((N, D)).astype(np.float32)
    if kind == 'peaked':                 # each query strongly matches one prefix key
        for r in range(N):
            K[rng.integers(0, P)] = q[r] * 2.5
    elif kind == 'two':                  # two prefix keys compete
        for r in range(N):
            j1, j2 = rng.integers(0, P, 2)
            K[j1] = q[r] * 2.0
            K[j2] = q[r] * 2.0 + 0.02 * rng.standard_normal(D)
    elif kind == 'sharp':                # large q: sharp attention everywhere
        q *= 4.0
    K, V, q = (bf16f(x) for x in (K, V, q))
    kc, kns = opaged.encode_cells('iso3', K[:P][:, None, :], quat=quat)
    vc, vns = opaged.encode_cells('iso3', V[:P][:, None, :], quat=quat)
    Kd = opaged.decode_cells('iso3', kc, kns, quat=quat, rotated=False)[:, 0]
    Vd = opaged.decode_cells('iso3', vc, vns, quat=quat, rotated=False)[:, 0]
    # codes as indices [P][D]
    def idx(codes):
        c = codes[:, 0]
        bits = np.unpackbits(c, axis=1, bitorder='little')
        return (bits.reshape(P, D, 3) * np.array([1, 2, 4])).sum(-1)
    kidx, vidx = idx(kc), idx(vc)
    kn_ = kns[:, 0, 0].astype(np.float32)
    vn_ = vns[:, 0, 0].astype(np.float32)
    sm = float(np.float32(1 / np.sqrt(D)))
    ref = reference(P, q, Kd, Vd, K[P:], V[P:], sm)
    res = {}
    for name, qp, wp, cwp in (('q2w2c2', 2, 2, 2), ('q1w2c2', 1, 2, 2), ('q2w1c2', 2, 1, 2), ('q1w1c2', 1, 1, 2),
                              ('q2w2c1', 2, 2, 1), ('q1w2c1', 1, 2, 1)):
        got = emulate(P, q, kidx, kn_, vidx, vn_, K[P:], V[P:], quat, sm, qp, wp, cwp)
        res[name] = float(np.max(np.abs(got - ref)))
    return res


if __name__ == '__main__':
    kinds = sys.argv[1:] or ['random', 'peaked', 'two', 'sharp']
    for kind in kinds:
        worst = {}
        for P in (1, 2, 5, 17, 64, 300, 2000):
            for seed in range(3):
                r = case(P, 48, 100 * P + seed, kind)
                for k, v in r.items():
                    worst[k] = max(worst.get(k, 0.0), v)
            print(kind, P, {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
