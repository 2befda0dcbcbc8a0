"""The five workload graphs, evaluated op by op on the CPU.

Test infrastructure only (see the package docstring).  Inputs are the
fp16/bf16 tensors drawn by ``workloads.generate``; they are upcast exactly
to fp32 and every op runs in fp32 (or ``dt``) with fp32 intermediates.
``mirror=True`` rounds each intermediate to the storage dtype the GPU path
writes it in; it separates rounding from bugs while debugging and is not the
graded oracle.

Row selection: for graphs whose rows are independent (every op acts row by
row), ``rows`` evaluates only those output rows, which is how full-size
outputs are sampled one by one.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import ops

F32 = np.float32


def _np(t: torch.Tensor, dt=F32) -> np.ndarray:
    return t.to(torch.float32).numpy().astype(dt, copy=False)


def _store(x: np.ndarray, tdt: torch.dtype, mirror: bool) -> np.ndarray:
    if not mirror:
        return x
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        tdt).to(torch.float32).numpy().astype(x.dtype, copy=False)


def mlp3(inp: Dict[str, torch.Tensor], rows: Optional[Sequence[int]] = None,
         mirror: bool = False, dt=F32) -> np.ndarray:
    """x <- relu(x @ W[i] + b[i]) for each layer i; the bias is a full
    [M, H] tensor per layer (no broadcasting) and the last layer also ends
    in ReLU.  MegaKittens Internals, section 02 (the traced MLP) and
    section 12 (binary ops do not broadcast, hence the (L, M, H) bias).
    """
    x = _np(inp["x"], dt)
    W = _np(inp["W"], dt)
    b = _np(inp["b"], dt)
    if rows is not None:
        x, b = x[list(rows)], b[:, list(rows)]
    for i in range(W.shape[0]):
        x = _store(ops.relu(ops.gemm(x, W[i], dt) + b[i]), torch.float16, mirror)
    return x


def decode(inp: Dict[str, torch.Tensor], dims: Dict[str, int],
           mirror: bool = False, dt=F32) -> np.ndarray:
    """One decoder layer at batch 1 as a chain of four GEMVs.

    qkv = rms(x, g1) @ Wqkv;  h = qkv[:, :n_q] @ Wo + x;
    gu = rms(h, g2) @ Wgu;  a = silu(gu[:, :I]) * gu[:, I:];  out = a @ Wd + h.

    "Implementing a Mega Kernel for B300", section 1 (the decoder-layer
    graph with gamma=, residual=, silu_mul= on the matmuls) and section 2
    (RMSNorm-input, residual and SiLU-mul fused as GEMV flags).  Reading:
    the attention call between QKV and O is omitted by the workload, so O
    reads the query slice of the QKV output.
    """
    bf = torch.bfloat16
    x = _np(inp["x"], dt)
    nq, I = dims["n_q"], dims["inter"]
    qkv = _store(ops.gemm(ops.rmsnorm(x, _np(inp["g1"], dt), dt=dt),
                          _np(inp["Wqkv"], dt), dt), bf, mirror)
    h = _store(ops.gemm(qkv[:, :nq], _np(inp["Wo"], dt), dt) + x, bf, mirror)
    gu = ops.gemm(ops.rmsnorm(h, _np(inp["g2"], dt), dt=dt), _np(inp["Wgu"], dt), dt)
    a = _store(ops.silu_mul(gu, I), bf, mirror)
    return ops.gemm(a, _np(inp["Wd"], dt), dt) + h


def prefill(inp: Dict[str, torch.Tensor], rows: Optional[Sequence[int]] = None,
            mirror: bool = False, dt=F32) -> np.ndarray:
    """Y = X @ W1 (stored fp16), Z = relu(Y @ W2).

    "Hand-writing a Blackwell GEMM", "Two workloads, not one" (the prefill
    shapes M = 8192 with attention-out and MLP-up N, K).
    """
    X = _np(inp["X"], dt)
    if rows is not None:
        X = X[list(rows)]
    Y = _store(ops.gemm(X, _np(inp["W1"], dt), dt), torch.float16, mirror)
    return ops.relu(ops.gemm(Y, _np(inp["W2"], dt), dt))


def decode_gemm(inp: Dict[str, torch.Tensor], dims: Dict[str, int],
                rows: Optional[Sequence[int]] = None, mirror: bool = False,
                dt=F32) -> np.ndarray:
    """Q = X0 @ Wqkv; A = Q[:, :n_q] @ Wo; U = A @ Wup; D = U @ Wdown.

    "Hand-writing a Blackwell GEMM", "Two workloads, not one" (the M = 256
    decode shapes: fused QKV, attention output, MLP up, MLP down).  Reading:
    with no attention op, attention-out reads the query slice of QKV.
    """
    f16 = torch.float16
    X = _np(inp["X0"], dt)
    if rows is not None:
        X = X[list(rows)]
    Q = _store(ops.gemm(X, _np(inp["Wqkv"], dt), dt), f16, mirror)
    A = _store(ops.gemm(Q[:, :dims["n_q"]], _np(inp["Wo"], dt), dt), f16, mirror)
    U = _store(ops.gemm(A, _np(inp["Wup"], dt), dt), f16, mirror)
    return ops.gemm(U, _np(inp["Wdown"], dt), dt)


def layer(inp: Dict[str, torch.Tensor], dims: Dict[str, int],
          mirror: bool = False, dt=F32, return_parts: bool = False):
    """Llama-style decoder layer prefill with causal grouped-query attention.

    xn = rms(x, g1); qkv = xn @ Wqkv; q, k, v = column slices of qkv,
    head-major [Q | K | V]; q, k <- rope(q, k) at positions 0..S-1;
    o = causal GQA attention(q, k, v); h1 = o @ Wo + x;
    gu = rms(h1, g2) @ Wgu; a = silu(gu[:, :I]) * gu[:, I:]; out = a @ Wd + h1.

    "Beating torch.compile with Megakernels", "Model Architecture" and the
    op list of its megakernel (RMS, QKV, ATTN, OUT, UP, GATE, DOWN);
    MegaKittens Internals section 14 (attention, BSHD, scale 1/sqrt(128)).
    """
    bf = torch.bfloat16
    S = dims["seq"]
    Hq, Hkv, d, I = dims["heads"], dims["kv_heads"], dims["head_dim"], dims["inter"]
    x = _np(inp["x"], dt)
    xn = _store(ops.rmsnorm(x, _np(inp["g1"], dt), dt=dt), bf, mirror)
    qkv = ops.gemm(xn, _np(inp["Wqkv"], dt), dt)
    q = qkv[:, :Hq * d].reshape(S, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(S, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(S, Hkv, d)
    q = _store(ops.rope(q, dt=dt), bf, mirror)
    k = _store(ops.rope(k, dt=dt), bf, mirror)
    v = _store(v, bf, mirror)
    o = _store(ops.causal_gqa_attention(q, k, v, True, dt).reshape(S, Hq * d),
               bf, mirror)
    h1 = _store(ops.gemm(o, _np(inp["Wo"], dt), dt) + x, bf, mirror)
    hn = _store(ops.rmsnorm(h1, _np(inp["g2"], dt), dt=dt), bf, mirror)
    gu = ops.gemm(hn, _np(inp["Wgu"], dt), dt)
    a = _store(ops.silu_mul(gu, I), bf, mirror)
    out = ops.gemm(a, _np(inp["Wd"], dt), dt) + h1
    if return_parts:
        return out, dict(xn=xn, q=q, k=k, v=v, o=o, h1=h1, hn=hn, a=a)
    return out


def decode_kv(inp: Dict[str, torch.Tensor], dims: Dict[str, int],
              mirror: bool = False, dt=F32, return_cache: bool = False):
    """The batch-1 decoder layer with its attention over a KV cache.

    qkv = rms(x, g1) @ Wqkv; q, k, v = the [Q | K | V] column blocks;
    o = decode_attention(q, k, v, caches, pos) (rotary at position pos, the
    new k and v appended as cache row pos, stored in the caches' bf16);
    h = o @ Wo + x; gu = rms(h, g2) @ Wgu; a = silu(gu[:, :I]) * gu[:, I:];
    out = a @ Wd + h.  "Implementing a Mega Kernel for B300", section 1 (the
    decoder layer's ops: RMS + QKV, RoPE + append, attention, O + residual,
    RMS + gate_up with SiLU-mul, down + residual).
    """
    bf = torch.bfloat16
    nq, nkv, hd, I = dims["n_q"], dims["n_kv"], dims["head_dim"], dims["inter"]
    Hq, Hkv = nq // hd, nkv // hd
    pos = int(inp["pos"].reshape(-1)[0])
    x = _np(inp["x"], dt)
    qkv = _store(ops.gemm(ops.rmsnorm(x, _np(inp["g1"], dt), dt=dt),
                          _np(inp["Wqkv"], dt), dt), bf, mirror)
    q = qkv[0, :nq].reshape(Hq, hd)
    k = qkv[0, nq:nq + nkv].reshape(Hkv, hd)
    v = qkv[0, nq + nkv:].reshape(Hkv, hd)
    kc = _np(inp["k_cache"], dt).reshape(-1, Hkv, hd)
    vc = _np(inp["v_cache"], dt).reshape(-1, Hkv, hd)
    def bf16(z):
        return torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).to(bf).to(
            torch.float32).numpy().astype(dt, copy=False)
    o, krow, vrow = ops.decode_attention(q, k, v, kc, vc, pos, dt=dt, round_kv=bf16)
    o = _store(o.reshape(1, nq), bf, mirror)
    h = _store(ops.gemm(o, _np(inp["Wo"], dt), dt) + x, bf, mirror)
    gu = ops.gemm(ops.rmsnorm(h, _np(inp["g2"], dt), dt=dt), _np(inp["Wgu"], dt), dt)
    a = _store(ops.silu_mul(gu, I), bf, mirror)
    out = ops.gemm(a, _np(inp["Wd"], dt), dt) + h
    if return_cache:
        return out, dict(k_row=krow.reshape(-1), v_row=vrow.reshape(-1), o=o, qkv=qkv)
    return out


def run(workload: str, inp: Dict[str, torch.Tensor], dims: Dict[str, int],
        rows: Optional[Sequence[int]] = None, mirror: bool = False,
        dt=F32) -> np.ndarray:
    """Evaluate a workload's graph output (optionally only ``rows``)."""
    if workload == "mlp3":
        return mlp3(inp, rows, mirror, dt)
    if workload == "decode":
        return decode(inp, dims, mirror, dt)
    if workload == "prefill":
        return prefill(inp, rows, mirror, dt)
    if workload == "decode_gemm":
        return decode_gemm(inp, dims, rows, mirror, dt)
    if workload == "layer":
        out = layer(inp, dims, mirror, dt)
        return out if rows is None else out[list(rows)]
    if workload == "decode_kv":
        return decode_kv(inp, dims, mirror, dt)
    raise KeyError(workload)


def flops(workload: str, dims: Dict[str, int]) -> int:
    """Algorithmic flops: 2*M*N*K per GEMM plus 4*H*d*S(S+1)/2 for causal
    attention; norms, softmax and elementwise ops are not counted."""
    d = dims
    if workload == "mlp3":
        return d["layers"] * 2 * d["m"] * d["h"] * d["h"]
    if workload == "decode":
        H, nq, nkv, I, M = d["hidden"], d["n_q"], d["n_kv"], d["inter"], d["m"]
        return 2 * M * (H * (nq + 2 * nkv) + nq * H + H * 2 * I + I * H)
    if workload == "prefill":
        return 2 * d["m"] * d["k"] * (d["n1"] + 0) + 2 * d["m"] * d["n1"] * d["n2"]
    if workload == "decode_gemm":
        M, K = d["m"], d["k"]
        return 2 * M * (K * d["n_qkv"] + d["n_q"] * d["n_o"] + d["n_o"] * d["n_up"]
                        + d["n_up"] * d["n_down"])
    if workload == "layer":
        S, H, Hq, Hkv, hd, I = (d["seq"], d["hidden"], d["heads"], d["kv_heads"],
                                d["head_dim"], d["inter"])
        lin = 2 * S * (H * (Hq + 2 * Hkv) * hd + Hq * hd * H + H * 2 * I + I * H)
        return lin + 4 * Hq * hd * S * (S + 1) // 2
    raise KeyError(workload)
