"""Op definitions of the oracle (numpy, fp32 by default).

Test infrastructure only (see the package docstring).  Each function is the
plain definition of the op, written out; no blocking, fusion or reordering.
Pass ``dt=np.float64`` for a higher-precision evaluation.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def gemm(a: np.ndarray, w: np.ndarray, dt=F32) -> np.ndarray:
    """y = a @ w with a [M, K], w [K, N] (weights stored K-major).

    MegaKittens Internals, section 02: the traced MLP calls ``aten.mm(x,
    select(W))`` with W indexed by layer, i.e. x @ W[i] with W[i] of shape
    [K, N].  Pinned by brute-force triple loops and permutation identities.
    """
    return np.matmul(a.astype(dt), w.astype(dt))


def relu(z: np.ndarray) -> np.ndarray:
    """max(z, 0).  MegaKittens Internals, section 02 (``aten.relu``)."""
    return np.maximum(z, 0)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z)).

    "Implementing a Mega Kernel for B300", section 2: the gate/up GEMV's
    SiLU-mul flag.  exp overflow for very negative z gives z/inf = -0, the
    correct limit.
    """
    with np.errstate(over="ignore"):
        return z / (1 + np.exp(-z))


def silu_mul(gu: np.ndarray, n: int) -> np.ndarray:
    """silu(gate) * up where gate = gu[:, :n], up = gu[:, n:2n].

    The gate half comes first ("Implementing a Mega Kernel for B300",
    section 1, the gate_up matmul with ``silu_mul=True``; the page names the
    two halves in that order only).
    """
    return silu(gu[:, :n]) * gu[:, n:2 * n]


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-6,
            dt=F32) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis.

    MegaKittens Internals, section 12 (RMSNorm: rows normalised, weight
    applied, EPS fixed at 1e-6).
    """
    x = x.astype(dt)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + dt(eps)) * gamma.astype(dt)


def rope_tables(n_pos: int, head_dim: int, theta: float = 10000.0):
    """cos/sin of p * theta^(-2i/head_dim) for p < n_pos, i < head_dim/2.

    Computed in float64.  The pages name rotary embedding without a formula
    ("Beating torch.compile with Megakernels", "Model Architecture";
    "Implementing a Mega Kernel for B300", the OpId table).  Reading: base
    10000, rotate-half pairing (i, i + head_dim/2).  Parity unpinned for the
    base and the pairing; the invariants (identity at p = 0, norm kept,
    relative-position inner products) are pinned.
    """
    half = head_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(u: np.ndarray, pos0: int = 0, theta: float = 10000.0,
         dt=F32) -> np.ndarray:
    """Rotate-half rotary embedding of u [S, heads, head_dim] at positions
    pos0 .. pos0+S-1.

    u'[i] = u[i] cos - u[i+h] sin,  u'[i+h] = u[i+h] cos + u[i] sin,
    with h = head_dim/2 and angle p * theta^(-2i/head_dim).
    """
    S, _, d = u.shape
    half = d // 2
    c, s = rope_tables(pos0 + S, d, theta)
    c = c[pos0:, None, :].astype(dt)
    s = s[pos0:, None, :].astype(dt)
    u = u.astype(dt)
    lo, hi = u[..., :half], u[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         causal: bool = True, dt=F32) -> np.ndarray:
    """Softmax attention per query head, q [S, Hq, d], k/v [S, Hkv, d].

    Query head h reads kv head h // (Hq / Hkv).  Scores are scaled by
    1/sqrt(d); with ``causal`` key j is visible to query i iff j <= i.
    The softmax subtracts the row max before exp.  MegaKittens Internals,
    section 14 (fixed 1/sqrt(128) scale, causal mask of col > row, BSHD);
    the TileLang tutorial's flash-attention mask keeps i >= j.  Evaluated
    densely per head: the plain definition, no online rescaling.
    """
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    scale = dt(1.0 / np.sqrt(d))
    out = np.empty((S, Hq, d), dtype=dt)
    mask = np.triu(np.ones((S, S), dtype=bool), k=1) if causal else None
    for h in range(Hq):
        kh = h // group
        sc = (q[:, h, :].astype(dt) @ k[:, kh, :].astype(dt).T) * scale
        if causal:
            sc = np.where(mask, -np.inf, sc)
        m = np.max(sc, axis=1, keepdims=True)
        p = np.exp(sc - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kh, :].astype(dt)
    return out


def decode_attention(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                     k_cache: np.ndarray, v_cache: np.ndarray, pos: int,
                     theta: float = 10000.0, dt=F32, round_kv=None):
    """Attention of one new token over a KV cache, q [Hq, d], k_new and
    v_new [Hkv, d], caches [S_max, Hkv, d], position p = pos.

    The new token's query and key are rotated at position p (``rope``);
    its key and value join the cache as row p (``round_kv``, if given, is
    applied to the rotated key and the value first: the storage rounding of
    the append); then o[h] = sum over j <= p of softmax_j(q'_h . K_j /
    sqrt(d)) V_j with kv head h // (Hq / Hkv) -- the plain softmax over the
    p + 1 keys, no splitting.  "Implementing a Mega Kernel for B300",
    section 2 (decode attention over the cache after the rotary step that
    appends the current k, v).  Returns (o [Hq, d], k row p, v row p).
    """
    Hq, d = q.shape
    Hkv = k_new.shape[0]
    qr = rope(q[None].astype(dt), pos0=pos, theta=theta, dt=dt)[0]
    kr = rope(k_new[None].astype(dt), pos0=pos, theta=theta, dt=dt)[0]
    vr = v_new.astype(dt)
    if round_kv is not None:
        kr, vr = round_kv(kr), round_kv(vr)
    K = np.concatenate([k_cache[:pos].astype(dt), kr[None]], axis=0)   # [p + 1, Hkv, d]
    V = np.concatenate([v_cache[:pos].astype(dt), vr[None]], axis=0)
    scale = dt(1.0 / np.sqrt(d))
    o = np.empty((Hq, d), dtype=dt)
    group = Hq // Hkv
    for h in range(Hq):
        g = h // group
        sc = (K[:, g, :] @ qr[h]) * scale
        e = np.exp(sc - np.max(sc))
        o[h] = (e / np.sum(e)) @ V[:, g, :]
    return o, kr, vr
