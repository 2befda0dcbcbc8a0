"""Pins of the oracle's decode attention over a KV cache (CPU only).

* Against the causal attention of a whole sequence (itself pinned by brute
  force): the last row of causal_gqa_attention(rope(q), rope(k), v) equals
  decode attention at p = S - 1 with the cache holding rope(k)[:S-1] and
  v[:S-1].  A wrong rotary position, a missing or doubled new key, a key
  read past p or a wrong GQA map each break it.
* p = 0: the only key is the new one, so o = v_new exactly.
* Equal scores (zero keys): o is the mean of the values 0..p.
* Brute force with scalar loops on a tiny case.
* The append: the returned row p is the rotated k_new and v_new.
"""
import math

import numpy as np
import pytest

from oracle import ops

rng = np.random.default_rng(77)


@pytest.mark.parametrize("S,Hq,Hkv", [(9, 4, 2), (33, 8, 2), (5, 2, 2)])
def test_matches_last_row_of_causal_attention(S, Hq, Hkv):
    d = 16
    q = rng.standard_normal((S, Hq, d))
    k = rng.standard_normal((S, Hkv, d))
    v = rng.standard_normal((S, Hkv, d))
    full = ops.causal_gqa_attention(ops.rope(q, dt=np.float64), ops.rope(k, dt=np.float64), v,
                                    True, np.float64)
    kr = ops.rope(k, dt=np.float64)
    cache_k = np.zeros((S + 3, Hkv, d))
    cache_v = np.zeros((S + 3, Hkv, d))
    cache_k[:S - 1] = kr[:S - 1]
    cache_v[:S - 1] = v[:S - 1]
    cache_k[S:] = 100.0       # rows past p must not be read
    cache_v[S:] = 100.0
    o, krow, vrow = ops.decode_attention(q[S - 1], k[S - 1], v[S - 1], cache_k, cache_v, S - 1,
                                         dt=np.float64)
    np.testing.assert_allclose(o, full[S - 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(krow, kr[S - 1], rtol=1e-12, atol=1e-12)
    assert np.array_equal(vrow, v[S - 1])


def test_position_zero_gives_the_new_value():
    Hq, Hkv, d = 4, 2, 8
    q = rng.standard_normal((Hq, d))
    kn = rng.standard_normal((Hkv, d))
    vn = rng.standard_normal((Hkv, d))
    cache = rng.standard_normal((6, Hkv, d))
    o, _, _ = ops.decode_attention(q, kn, vn, cache, cache, 0, dt=np.float64)
    for h in range(Hq):
        assert np.array_equal(o[h], vn[h // 2])


def test_equal_scores_give_the_mean():
    Hq, Hkv, d, p = 6, 3, 8, 11
    q = rng.standard_normal((Hq, d))
    kn = np.zeros((Hkv, d))
    vn = rng.standard_normal((Hkv, d))
    kc = np.zeros((20, Hkv, d))
    vc = rng.standard_normal((20, Hkv, d))
    o, _, _ = ops.decode_attention(q, kn, vn, kc, vc, p, dt=np.float64)
    for h in range(Hq):
        g = h // 2
        want = (vc[:p, g].sum(axis=0) + vn[g]) / (p + 1)
        np.testing.assert_allclose(o[h], want, rtol=1e-12, atol=1e-12)


def test_brute_force_scalar_loops():
    Hq, Hkv, d, p = 2, 1, 4, 3
    q = rng.standard_normal((Hq, d))
    kn = rng.standard_normal((Hkv, d))
    vn = rng.standard_normal((Hkv, d))
    kc = rng.standard_normal((5, Hkv, d))
    vc = rng.standard_normal((5, Hkv, d))
    o, _, _ = ops.decode_attention(q, kn, vn, kc, vc, p, dt=np.float64)

    def rot(u, pos):
        h = d // 2
        out = [0.0] * d
        for i in range(h):
            th = pos * 10000.0 ** (-2.0 * i / d)
            out[i] = u[i] * math.cos(th) - u[i + h] * math.sin(th)
            out[i + h] = u[i + h] * math.cos(th) + u[i] * math.sin(th)
        return out
    kr = rot(kn[0], p)
    for h in range(Hq):
        qr = rot(q[h], p)
        keys = [list(kc[j, 0]) for j in range(p)] + [kr]
        vals = [list(vc[j, 0]) for j in range(p)] + [list(vn[0])]
        sc = [sum(a * b for a, b in zip(qr, kk)) / math.sqrt(d) for kk in keys]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = sum(e)
        for t in range(d):
            want = sum(e[j] * vals[j][t] for j in range(p + 1)) / z
            assert abs(o[h, t] - want) < 1e-12
