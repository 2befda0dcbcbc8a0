"""Pins of the oracle's op definitions against brute force, closed forms
and invariants (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import ops, graphs
import workloads

rng = np.random.default_rng(1234)


def brute_mm(a, b):
    M, K = a.shape
    N = b.shape[1]
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(a[i, k]) * float(b[k, j])
            out[i][j] = s
    return np.array(out)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 3, 13), (4, 130, 9),
                                   (64, 17, 3), (1, 64, 130)])
def test_gemm_brute_force(M, N, K):
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    ref = brute_mm(a, b)
    got = ops.gemm(a, b)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= 1e-6


def test_gemm_identity_and_permutation_bias_relu():
    M, H = 9, 12
    x = rng.standard_normal((M, H)).astype(np.float32)
    # W = I, b = 0 -> relu(x) exactly
    assert np.array_equal(ops.relu(ops.gemm(x, np.eye(H, dtype=np.float32)) + 0), ops.relu(x))
    # non-symmetric permutation P[k, perm[k]] = 1: (x P)[:, perm[k]] = x[:, k]
    perm = np.roll(np.arange(H), 3)
    P = np.zeros((H, H), np.float32)
    P[np.arange(H), perm] = 1
    xp = ops.gemm(x, P)
    expect = np.empty_like(x)
    expect[:, perm] = x
    assert np.array_equal(xp, expect)
    # and the transposed product is different (so a transposed W is caught)
    assert not np.array_equal(ops.gemm(x, P.T), expect)
    # b = -(x @ W) -> relu(x @ W + b) == 0
    W = rng.standard_normal((H, H)).astype(np.float32)
    y = ops.gemm(x, W)
    assert np.all(ops.relu(y + (-y)) == 0)
    # relu(y) - relu(-y) == y
    assert np.array_equal(ops.relu(y) - ops.relu(-y), y)


def test_residual_zero_weight():
    x = rng.standard_normal((5, 8)).astype(np.float32)
    r = rng.standard_normal((5, 6)).astype(np.float32)
    assert np.array_equal(ops.gemm(x, np.zeros((8, 6), np.float32)) + r, r)


def test_rmsnorm_closed_forms():
    H = 64
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    for c in (0.0, 1.0, -3.5, 1e-3):
        x = np.full((1, H), c, np.float32)
        expect = g * (c / math.sqrt(c * c + 1e-6))
        np.testing.assert_allclose(ops.rmsnorm(x, g)[0], expect, rtol=2e-6, atol=1e-7)
    x = rng.standard_normal((4, H)).astype(np.float32)
    for a in (0.5, 3.0, 100.0):
        np.testing.assert_allclose(ops.rmsnorm(a * x, g), ops.rmsnorm(x, g), rtol=1e-4)


def test_rmsnorm_brute_force():
    x = rng.standard_normal((3, 7))
    g = rng.standard_normal(7)
    got = ops.rmsnorm(x, g, dt=np.float64)
    for r in range(3):
        ms = sum(float(v) ** 2 for v in x[r]) / 7
        for c in range(7):
            assert abs(got[r, c] - x[r, c] / math.sqrt(ms + 1e-6) * g[c]) < 1e-12


def test_silu_and_silu_mul():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0, -200.0, 200.0], np.float64)
    got = ops.silu(z)
    for zi, gi in zip(z, got):
        assert abs(gi - zi / (1 + math.exp(-zi)) if zi > -700 else gi) < 1e-12
    assert got[0] == 0.0 and abs(got[3] - 30.0) < 1e-9 and abs(got[4]) < 1e-11
    gu = rng.standard_normal((3, 8)).astype(np.float32)
    z0 = gu.copy(); z0[:, :4] = 0
    assert np.all(ops.silu_mul(z0, 4) == 0)
    u0 = gu.copy(); u0[:, 4:] = 0
    assert np.all(ops.silu_mul(u0, 4) == 0)
    # gate half first: swapping halves changes the result
    sw = np.concatenate([gu[:, 4:], gu[:, :4]], 1)
    assert not np.allclose(ops.silu_mul(sw, 4), ops.silu_mul(gu, 4))


def _brute_attention(q, k, v, causal):
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((S, Hq, d))
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        for i in range(S):
            js = range(i + 1) if causal else range(S)
            sc = [sum(float(q[i, h, t]) * float(k[j, kh, t]) for t in range(d)) / math.sqrt(d)
                  for j in js]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for t in range(d):
                out[i, h, t] = sum(e[n] * float(v[j, kh, t]) for n, j in enumerate(js)) / z
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_attention_brute_force(causal):
    S, Hq, Hkv, d = 7, 4, 2, 8
    q = rng.standard_normal((S, Hq, d))
    k = rng.standard_normal((S, Hkv, d))
    v = rng.standard_normal((S, Hkv, d))
    got = ops.causal_gqa_attention(q, k, v, causal, dt=np.float64)
    np.testing.assert_allclose(got, _brute_attention(q, k, v, causal), rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    S, Hq, Hkv, d = 33, 8, 2, 16
    q = rng.standard_normal((S, Hq, d)).astype(np.float32)
    k = rng.standard_normal((S, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((S, Hkv, d)).astype(np.float32)
    o = ops.causal_gqa_attention(q, k, v)
    # row 0 sees only key 0
    for h in range(Hq):
        assert np.array_equal(o[0, h], v[0, h // 4])
    # equal scores -> running mean of v
    o0 = ops.causal_gqa_attention(q, np.zeros_like(k), v, dt=np.float64)
    cm = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, S + 1)[:, None, None]
    for h in range(Hq):
        np.testing.assert_allclose(o0[:, h], cm[:, h // 4], rtol=1e-12, atol=1e-12)
    # per-kv-head constant V pins the h // group mapping
    vc = np.broadcast_to(np.arange(1, Hkv + 1, dtype=np.float32)[None, :, None], v.shape)
    oc = ops.causal_gqa_attention(q, k, np.ascontiguousarray(vc))
    for h in range(Hq):
        np.testing.assert_allclose(oc[:, h], h // (Hq // Hkv) + 1, rtol=1e-5)


def test_rope_invariants():
    S, H, d = 40, 3, 128
    u = rng.standard_normal((S, H, d))
    r = ops.rope(u, dt=np.float64)
    # position 0 is the identity
    assert np.allclose(r[0], u[0], rtol=0, atol=0)
    # every (i, i + d/2) pair keeps its norm
    half = d // 2
    n0 = u[..., :half] ** 2 + u[..., half:] ** 2
    n1 = r[..., :half] ** 2 + r[..., half:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # <rope(q, m), rope(k, n)> depends only on m - n
    q = rng.standard_normal((1, 1, d))
    kk = rng.standard_normal((1, 1, d))
    def at(x, p):
        return ops.rope(np.repeat(x, p + 1, axis=0), dt=np.float64)[p, 0]
    a = at(q, 9) @ at(kk, 4)
    b = at(q, 25) @ at(kk, 20)
    assert abs(a - b) < 1e-10
    assert abs(a - at(q, 6) @ at(kk, 4)) > 1e-6


def test_graph_special_cases():
    d = workloads.small_dims("mlp3")
    inp = workloads.generate("mlp3", d)
    inp["W"] = torch.eye(d["h"], dtype=torch.float16).expand(3, -1, -1).contiguous()
    inp["b"] = torch.zeros_like(inp["b"])
    out = graphs.mlp3(inp)
    assert np.array_equal(out, np.maximum(inp["x"].float().numpy(), 0))
    # decode with Wo = 0 and Wd = 0 reduces to out = x
    d = workloads.small_dims("decode")
    inp = workloads.generate("decode", d)
    inp["Wo"].zero_(); inp["Wd"].zero_()
    assert np.array_equal(graphs.decode(inp, d), inp["x"].float().numpy())
    # layer with Wo = 0 and Wd = 0 reduces to out = x
    d = workloads.small_dims("layer")
    inp = workloads.generate("layer", d)
    inp["Wo"].zero_(); inp["Wd"].zero_()
    assert np.array_equal(graphs.layer(inp, d), inp["x"].float().numpy())


def test_row_selection_matches_full():
    for wl in ("mlp3", "prefill", "decode_gemm"):
        d = workloads.small_dims(wl)
        inp = workloads.generate(wl, d)
        full = graphs.run(wl, inp, d)
        rows = [0, 7, d["m"] - 1]
        np.testing.assert_allclose(graphs.run(wl, inp, d, rows=rows), full[rows],
                                   rtol=1e-5, atol=1e-5)


def test_flops_match_closed_forms():
    # Algorithmic flop counts per workload at full size (2*M*N*K per GEMM
    # plus 4*H*d*S(S+1)/2 for causal attention), in GFLOP.
    want = dict(mlp3=6.44, decode=0.44, prefill=4947.8, decode_gemm=317.8, layer=927.7)
    for wl, gf in want.items():
        got = graphs.flops(wl, workloads.default_dims(wl)) / 1e9
        assert abs(got - gf) / gf < 0.01, (wl, got)


def test_inputs_deterministic_and_distributed():
    a = workloads.generate("decode", workloads.small_dims("decode"))
    b = workloads.generate("decode", workloads.small_dims("decode"))
    for k in a:
        assert torch.equal(a[k], b[k])
    w = workloads.generate("prefill", dict(m=64, k=1024, n1=1024, n2=64))["W1"].float()
    assert abs(w.std().item() - 1 / 32) < 1e-3 and abs(w.mean().item()) < 1e-3
    g = a["g1"].float()
    assert abs(g.mean().item() - 1) < 0.01 and abs(g.std().item() - 0.02) < 0.005
