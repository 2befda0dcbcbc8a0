"""Pins of the oracle's graph wiring (CPU only).

Each workload graph in ``oracle.graphs`` is run on weights chosen so that
its output has a closed form, and that closed form is evaluated here with
scalar loops over Python floats (``math`` only, no oracle code).  The
weights are built so that a plausible miswiring gives a different answer:

* decode: O reads the query slice of qkv (the K|V columns hold other
  values), gate_up normalises h (not x) with gamma 2 (not gamma 1), the
  gate half comes first, down adds h (not x).
  ("Implementing a Mega Kernel for B300", section 1: the decoder-layer
  graph with gamma=, residual= and silu_mul= on its matmuls.)
* layer: K and V come from their own column blocks of Wqkv in [Q | K | V]
  order, q and k are rotated and v is not, O adds x, gate_up normalises h1,
  down adds h1.  ("Beating torch.compile with Megakernels in CuTe DSL",
  "Model Architecture".)
* prefill: ReLU only on the second product.  ("Hand-writing a Blackwell
  GEMM", "Two workloads, not one".)
* decode_gemm: attention-out reads the query slice of the QKV output.
* decode_kv: attention over the cache reads the V block, cache rows below
  the position and the appended new value, then the decode wiring.
* silu_mul: silu of the gate half times the up half.
"""
import math

import numpy as np
import torch

import workloads
from oracle import graphs, ops


def _silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def _rms_row(x, g, eps=1e-6):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gg for v, gg in zip(x, g)]


def _close(got, want, rtol=2e-5, atol=2e-6):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} elements off, first {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def test_silu_mul_gate_then_up():
    z, u = 1.5, -2.0
    got = ops.silu_mul(np.array([[z, u]], np.float64), 1)
    assert abs(got[0, 0] - _silu(z) * u) < 1e-14
    # the swapped reading silu(u) * z gives a different number here
    assert abs(_silu(u) * z - _silu(z) * u) > 0.1


def _gamma(H, base, step):
    # bf16-exact values, a different one per column
    return torch.tensor([base + step * (i % 4) for i in range(H)], dtype=torch.bfloat16)


def test_decode_wiring_closed_form():
    H, nkv = 64, 16
    d = dict(m=1, hidden=H, n_q=H, n_kv=nkv, inter=H)
    inp = workloads.generate("decode", d)
    s, c = 2.0, 0.5
    bf = torch.bfloat16
    Wqkv = torch.zeros(H, H + 2 * nkv, dtype=bf)
    Wqkv[:, :H] = s * torch.eye(H, dtype=bf)
    # the K|V columns hold values a slice reading them would pick up
    Wqkv[:, H:] = torch.randn(H, 2 * nkv, generator=torch.Generator().manual_seed(5)).to(bf)
    inp["Wqkv"] = Wqkv
    inp["Wo"] = torch.eye(H, dtype=bf)
    inp["Wgu"] = torch.cat([c * torch.eye(H, dtype=bf), torch.eye(H, dtype=bf)], 1)
    inp["Wd"] = torch.eye(H, dtype=bf)
    inp["g1"] = _gamma(H, 1.0, 0.25)
    inp["g2"] = _gamma(H, 0.5, 0.5)
    x = [float(v) for v in inp["x"][0].float()]
    g1 = [float(v) for v in inp["g1"].float()]
    g2 = [float(v) for v in inp["g2"].float()]
    xn = _rms_row(x, g1)
    h = [s * a + b for a, b in zip(xn, x)]
    hn = _rms_row(h, g2)
    out = [_silu(c * v) * v + hh for v, hh in zip(hn, h)]
    _close(graphs.decode(inp, d)[0], out)


def test_prefill_relu_on_second_product_only():
    m, k = 6, 16
    n1, n2 = 16, 24
    d = dict(m=m, k=k, n1=n1, n2=n2)
    inp = workloads.generate("prefill", d)
    tau = [(3 * i + 1) % n1 for i in range(k)]          # W1 column of row i
    sig = [(5 * j + 2) % n2 for j in range(n1)]         # W2 column of row j (injective)
    W1 = torch.zeros(k, n1, dtype=torch.float16)
    W2 = torch.zeros(n1, n2, dtype=torch.float16)
    for i in range(k):
        W1[i, tau[i]] = -1.0
    for j in range(n1):
        W2[j, sig[j]] = -1.0
    inp["W1"], inp["W2"] = W1, W2
    X = inp["X"].float().tolist()
    want = [[0.0] * n2 for _ in range(m)]
    for r in range(m):
        for i in range(k):
            # Y[r, tau[i]] = -X[r, i]; Z[r, sig[tau[i]]] = relu(X[r, i])
            want[r][sig[tau[i]]] = max(X[r][i], 0.0)
    _close(graphs.prefill(inp), want, rtol=0, atol=0)
    # a ReLU on Y as well would zero every output here: the pin tells them apart
    assert np.count_nonzero(np.asarray(want)) > 0


def test_decode_gemm_attention_out_reads_query_slice():
    d = dict(m=4, k=16, n_qkv=24, n_q=16, n_o=16, n_up=32, n_down=16)
    inp = workloads.generate("decode_gemm", d)
    f16 = torch.float16
    p1 = [(7 * i + 3) % 16 for i in range(16)]
    Wqkv = torch.zeros(16, 24, dtype=f16)
    for i in range(16):
        Wqkv[i, p1[i]] = 1.0
    # K|V columns of the QKV output: non-zero, so reading them changes A
    Wqkv[:, 16:] = torch.randn(16, 8, generator=torch.Generator().manual_seed(2)).to(f16)
    p2 = [(5 * i + 1) % 16 for i in range(16)]
    Wo = torch.zeros(16, 16, dtype=f16)
    for i in range(16):
        Wo[i, p2[i]] = 1.0
    up = [2 * i + 1 for i in range(16)]              # A col i -> U col 2i+1
    Wup = torch.zeros(16, 32, dtype=f16)
    for i in range(16):
        Wup[i, up[i]] = 1.0
    Wdn = torch.zeros(32, 16, dtype=f16)
    for i in range(16):
        Wdn[up[i], (i + 9) % 16] = 1.0
    inp.update(Wqkv=Wqkv, Wo=Wo, Wup=Wup, Wdown=Wdn)
    X = inp["X0"].float().tolist()
    want = [[0.0] * 16 for _ in range(4)]
    for r in range(4):
        for i in range(16):
            # Q[:, p1[i]] = X[:, i]; A[:, p2[q]] = Q[:, q]; D[:, (a + 9) % 16] = A[:, a]
            a = p2[p1[i]]
            want[r][(a + 9) % 16] = X[r][i]
    _close(graphs.decode_gemm(inp, d), want, rtol=0, atol=0)


def _rope_pair_norms(u):
    half = u.shape[-1] // 2
    return u[..., :half] ** 2 + u[..., half:] ** 2


def test_layer_wiring_closed_form():
    S, H, Hq, Hkv, hd, I = 8, 256, 2, 1, 128, 384
    d = dict(seq=S, hidden=H, heads=Hq, kv_heads=Hkv, head_dim=hd, inter=I)
    inp = workloads.generate("layer", d)
    bf = torch.bfloat16
    nq, nkv = Hq * hd, Hkv * hd
    gen = torch.Generator().manual_seed(9)
    # Wqkv = [A | B | C]: q, k and v select different columns of xn
    colsA = [(3 * j + 1) % H for j in range(nq)]
    colsB = [(5 * j + 7) % H for j in range(nkv)]
    colsC = [(7 * j + 2) % H for j in range(nkv)]
    Wqkv = torch.zeros(H, nq + 2 * nkv, dtype=bf)
    for j, c in enumerate(colsA):
        Wqkv[c, j] = 1.0
    for j, c in enumerate(colsB):
        Wqkv[c, nq + j] = 1.0
    for j, c in enumerate(colsC):
        Wqkv[c, nq + nkv + j] = 1.0
    inp["Wqkv"] = Wqkv
    inp["Wo"] = torch.eye(nq, H, dtype=bf)                  # h1 = o + x (nq == H)
    cg = 0.5
    Wgu = torch.zeros(H, 2 * I, dtype=bf)
    Wgu[:, :H] = cg * torch.eye(H, dtype=bf)                # gate[:, :H] = cg * hn
    Wgu[:, I:I + H] = torch.eye(H, dtype=bf)                # up[:, :H] = hn
    inp["Wgu"] = Wgu
    inp["Wd"] = torch.eye(I, H, dtype=bf)                   # out = a[:, :H] + h1
    inp["g1"] = _gamma(H, 1.0, 0.25)
    inp["g2"] = _gamma(H, 0.5, 0.5)
    out, parts = graphs.layer(inp, d, return_parts=True)
    x = inp["x"].float().tolist()
    g1 = [float(v) for v in inp["g1"].float()]
    g2 = [float(v) for v in inp["g2"].float()]
    xn = [_rms_row(r, g1) for r in x]
    _close(parts["xn"], xn)
    # V: the C block, not rotated at any position
    v_want = [[[xn[s][colsC[j]] for j in range(nkv)]] for s in range(S)]
    _close(parts["v"], v_want)
    # K: the B block; rotation is the identity at position 0 and keeps each
    # (i, i + hd/2) pair's norm elsewhere
    k_unrot = np.array([[[xn[s][colsB[j]] for j in range(nkv)]] for s in range(S)])
    _close(parts["k"][0], k_unrot[0])
    _close(_rope_pair_norms(parts["k"]), _rope_pair_norms(k_unrot), rtol=1e-4, atol=1e-5)
    assert np.abs(parts["k"][1:] - k_unrot[1:]).max() > 1e-3   # rotated past position 0
    q_unrot = np.array([[[xn[s][colsA[h * hd + j]] for j in range(hd)] for h in range(Hq)]
                        for s in range(S)])
    _close(parts["q"][0], q_unrot[0])
    _close(_rope_pair_norms(parts["q"]), _rope_pair_norms(q_unrot), rtol=1e-4, atol=1e-5)
    assert np.abs(parts["q"][1:] - q_unrot[1:]).max() > 1e-3
    # residual and norm sources
    o = parts["o"].reshape(S, nq).astype(np.float64).tolist()
    h1 = [[o[s][c] + x[s][c] for c in range(H)] for s in range(S)]
    _close(parts["h1"], h1)
    hn = [_rms_row(r, g2) for r in h1]
    _close(parts["hn"], hn, rtol=1e-4, atol=1e-5)
    a_want = [[(_silu(cg * hn[s][c]) * hn[s][c] if c < H else 0.0) for c in range(I)] for s in range(S)]
    _close(parts["a"], a_want, rtol=1e-4, atol=1e-5)
    out_want = [[a_want[s][c] + h1[s][c] for c in range(H)] for s in range(S)]
    _close(out, out_want, rtol=1e-4, atol=1e-5)


def test_mlp3_bias_before_relu_every_layer():
    # W[i] = I, b[i] = -x_i: every layer's pre-activation is exactly 0, so a
    # bias added after the ReLU (relu(x) - x) or a missing last ReLU would
    # leave non-zero outputs; b = +1 with W = I gives x + 3 past the first
    # layer's relu for positive x.
    d = dict(layers=3, m=4, h=8)
    inp = workloads.generate("mlp3", d)
    f16 = torch.float16
    inp["W"] = torch.eye(8, dtype=f16).expand(3, -1, -1).contiguous()
    b = torch.zeros(3, 4, 8, dtype=f16)
    b[0] = -inp["x"]
    inp["b"] = b
    assert np.array_equal(graphs.mlp3(inp), np.zeros((4, 8), np.float32))
    inp["b"] = torch.full((3, 4, 8), 1.0, dtype=f16)
    x = inp["x"].float().tolist()
    want = []
    for r in x:
        row = []
        for v in r:
            y = max(v + 1.0, 0.0)
            y = max(y + 1.0, 0.0)
            row.append(max(y + 1.0, 0.0))
        want.append(row)
    _close(graphs.mlp3(inp), want, rtol=1e-6, atol=1e-6)


def test_decode_kv_wiring_closed_form():
    # q = k = 0 (their Wqkv blocks are zero) makes every score equal, so each
    # head's attention output is the mean of its kv head's cache values 0..p-1
    # and the new value; v_new selects the first n_kv columns of xn.  Pins:
    # attention reads the V block (not K), cache rows below p only, the new
    # value as row p, the GQA map, then O + x, gate_up on h, down + h.
    H, hd, Hq, Hkv, I, Smax, p = 16, 8, 2, 1, 16, 7, 4
    nq, nkv = Hq * hd, Hkv * hd
    d = dict(m=1, hidden=H, n_q=nq, n_kv=nkv, head_dim=hd, inter=I, s_max=Smax, pos=p)
    inp = workloads.generate("decode_kv", d)
    bf = torch.bfloat16
    Wqkv = torch.zeros(H, nq + 2 * nkv, dtype=bf)
    Wqkv[:nkv, nq + nkv:] = torch.eye(nkv, dtype=bf)
    inp["Wqkv"] = Wqkv
    inp["Wo"] = torch.eye(nq, H, dtype=bf)
    c = 0.5
    inp["Wgu"] = torch.cat([c * torch.eye(H, I, dtype=bf), torch.eye(H, I, dtype=bf)], 1)
    inp["Wd"] = torch.eye(I, H, dtype=bf)
    inp["g1"] = _gamma(H, 1.0, 0.25)
    inp["g2"] = _gamma(H, 0.5, 0.5)
    vc = inp["v_cache"].float().tolist()
    x = [float(v) for v in inp["x"][0].float()]
    xn = _rms_row(x, [float(v) for v in inp["g1"].float()])
    # the appended value is stored in the cache's bf16
    vnew = [float(torch.tensor(v).to(bf).float()) for v in xn[:nkv]]
    mean = [(sum(vc[j][t] for j in range(p)) + vnew[t]) / (p + 1) for t in range(nkv)]
    o = mean * Hq                              # every query head reads kv head 0
    h = [a + b for a, b in zip(o, x)]
    hn = _rms_row(h, [float(v) for v in inp["g2"].float()])
    out = [_silu(c * v) * v + hh for v, hh in zip(hn, h)]
    _close(graphs.decode_kv(inp, d)[0], out, rtol=1e-4, atol=1e-4)
