"""Seeded synthetic inputs for the five tile-graph workloads.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``tiled_gemm_graph_amd``).  It holds *data only*: tensor names, shapes,
dtypes, the normal distribution each tensor is drawn from, and the seeded
draw itself.  It contains none of the method's arithmetic (no GEMM, norm,
attention, tiling or scheduling), so sharing it does not couple the two
implementations.

Draw recipe (identical for every workload):

* one CPU ``torch.Generator`` seeded with ``seed`` (default 0),
* tensors drawn in the order listed by :func:`spec`, each as
  ``torch.randn(shape, dtype=float32, generator=g) * std + mean``,
* then rounded once to the storage dtype (fp16 or bf16) with ``.to()``,
  which rounds to nearest even.

Both sides consume the resulting fp16/bf16 bytes; the oracle upcasts them.

Workloads (full sizes; ``dims`` overrides give the small parity sizes):

``mlp3``        3-layer MLP x = relu(x @ W[i] + b[i]), fp16.  MegaKittens
                Internals, section 02 (the traced test MLP) and section 04.
``decode``      one decoder layer at batch 1 as a GEMV chain, bf16.
                "Implementing a Mega Kernel for B300", section 1 (the
                decoder-layer graph) and section 2 (fused GEMV flags).
``prefill``     two chained fp16 GEMMs X@W1 -> Y, relu(Y@W2), M=8192.
                "Hand-writing a Blackwell GEMM", "Two workloads, not one".
``decode_gemm`` four chained fp16 GEMMs at M=256 (Llama-3-70B linear
                shapes).  Same page and section.
``layer``       a Llama-style decoder layer prefill with causal GQA
                attention, bf16.  "Beating torch.compile with Megakernels",
                "Model Architecture"; MegaKittens Internals section 14.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import torch

WORKLOADS = ("mlp3", "decode", "prefill", "decode_gemm", "layer")
# graphs beyond the five configurations (built on them)
EXTRA_WORKLOADS = ("decode_kv",)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    dtype: torch.dtype
    mean: float
    std: float


def default_dims(workload: str) -> Dict[str, int]:
    """Full-size dimensions of a workload."""
    if workload == "mlp3":
        return dict(layers=3, m=1024, h=1024)
    if workload == "decode":
        return dict(m=1, hidden=4096, n_q=4096, n_kv=1024, inter=14336)
    if workload == "prefill":
        return dict(m=8192, k=8192, n1=8192, n2=28672)
    if workload == "decode_gemm":
        return dict(m=256, k=8192, n_qkv=10240, n_q=8192, n_o=8192,
                    n_up=28672, n_down=8192)
    if workload == "layer":
        return dict(seq=2048, hidden=4096, heads=32, kv_heads=8,
                    head_dim=128, inter=14336)
    if workload == "decode_kv":
        return dict(m=1, hidden=4096, n_q=4096, n_kv=1024, head_dim=128, inter=14336,
                    s_max=4096, pos=4095)
    raise KeyError(workload)


def small_dims(workload: str) -> Dict[str, int]:
    """Reduced sizes the oracle finishes in seconds.

    They still span several tiles per node and leave a ragged tail in M
    where the method allows one.
    """
    if workload == "mlp3":
        return dict(layers=3, m=200, h=256)
    if workload == "decode":
        return dict(m=1, hidden=512, n_q=512, n_kv=128, inter=768)
    if workload == "prefill":
        return dict(m=200, k=256, n1=384, n2=512)
    if workload == "decode_gemm":
        return dict(m=48, k=512, n_qkv=768, n_q=512, n_o=512,
                    n_up=1024, n_down=512)
    if workload == "layer":
        return dict(seq=320, hidden=512, heads=4, kv_heads=1,
                    head_dim=128, inter=768)
    if workload == "decode_kv":
        return dict(m=1, hidden=512, n_q=512, n_kv=256, head_dim=128, inter=768,
                    s_max=384, pos=200)
    raise KeyError(workload)


def spec(workload: str, dims: Dict[str, int] | None = None) -> List[TensorSpec]:
    """Tensors of a workload in draw order."""
    d = dict(default_dims(workload))
    if dims:
        d.update(dims)
    f16, bf16 = torch.float16, torch.bfloat16
    if workload == "mlp3":
        L, M, H = d["layers"], d["m"], d["h"]
        return [
            TensorSpec("x", (M, H), f16, 0.0, 1.0),
            TensorSpec("W", (L, H, H), f16, 0.0, 1.0 / 32.0),
            TensorSpec("b", (L, M, H), f16, 0.0, 0.1),
        ]
    if workload == "decode":
        M, H = d["m"], d["hidden"]
        nqkv = d["n_q"] + 2 * d["n_kv"]
        I = d["inter"]
        return [
            TensorSpec("x", (M, H), bf16, 0.0, 1.0),
            TensorSpec("g1", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wqkv", (H, nqkv), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wo", (d["n_q"], H), bf16, 0.0, 1.0 / math.sqrt(d["n_q"])),
            TensorSpec("g2", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wgu", (H, 2 * I), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wd", (I, H), bf16, 0.0, 1.0 / math.sqrt(I)),
        ]
    if workload == "prefill":
        M, K, N1, N2 = d["m"], d["k"], d["n1"], d["n2"]
        return [
            TensorSpec("X", (M, K), f16, 0.0, 1.0),
            TensorSpec("W1", (K, N1), f16, 0.0, 1.0 / math.sqrt(K)),
            TensorSpec("W2", (N1, N2), f16, 0.0, 1.0 / math.sqrt(N1)),
        ]
    if workload == "decode_gemm":
        M, K = d["m"], d["k"]
        return [
            TensorSpec("X0", (M, K), f16, 0.0, 1.0),
            TensorSpec("Wqkv", (K, d["n_qkv"]), f16, 0.0, 1.0 / math.sqrt(K)),
            TensorSpec("Wo", (d["n_q"], d["n_o"]), f16, 0.0, 1.0 / math.sqrt(d["n_q"])),
            TensorSpec("Wup", (d["n_o"], d["n_up"]), f16, 0.0, 1.0 / math.sqrt(d["n_o"])),
            TensorSpec("Wdown", (d["n_up"], d["n_down"]), f16, 0.0,
                       1.0 / math.sqrt(d["n_up"])),
        ]
    if workload == "decode_kv":
        M, H, I, Smax = d["m"], d["hidden"], d["inter"], d["s_max"]
        nqkv = d["n_q"] + 2 * d["n_kv"]
        return [
            TensorSpec("x", (M, H), bf16, 0.0, 1.0),
            TensorSpec("g1", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wqkv", (H, nqkv), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wo", (d["n_q"], H), bf16, 0.0, 1.0 / math.sqrt(d["n_q"])),
            TensorSpec("g2", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wgu", (H, 2 * I), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wd", (I, H), bf16, 0.0, 1.0 / math.sqrt(I)),
            # the cache holds rotated keys and values of earlier tokens:
            # drawn i.i.d. N(0, 1), the scale of a projected activation
            TensorSpec("k_cache", (Smax, d["n_kv"]), bf16, 0.0, 1.0),
            TensorSpec("v_cache", (Smax, d["n_kv"]), bf16, 0.0, 1.0),
            # the position of the new token: a constant, no draw
            TensorSpec("pos", (1,), torch.int32, float(d["pos"]), 0.0),
        ]
    if workload == "layer":
        S, H = d["seq"], d["hidden"]
        nq = d["heads"] * d["head_dim"]
        nkv = d["kv_heads"] * d["head_dim"]
        I = d["inter"]
        return [
            TensorSpec("x", (S, H), bf16, 0.0, 1.0),
            TensorSpec("g1", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wqkv", (H, nq + 2 * nkv), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wo", (nq, H), bf16, 0.0, 1.0 / math.sqrt(nq)),
            TensorSpec("g2", (H,), bf16, 1.0, 0.02),
            TensorSpec("Wgu", (H, 2 * I), bf16, 0.0, 1.0 / math.sqrt(H)),
            TensorSpec("Wd", (I, H), bf16, 0.0, 1.0 / math.sqrt(I)),
        ]
    raise KeyError(workload)


def dims_of(workload: str, dims: Dict[str, int] | None = None) -> Dict[str, int]:
    d = dict(default_dims(workload))
    if dims:
        d.update(dims)
    return d


_CHUNK = 1 << 24  # elements drawn per randn call; bounds the fp32 temporary


def _draw(ts: TensorSpec, g: torch.Generator) -> torch.Tensor:
    n = 1
    for s in ts.shape:
        n *= s
    if not ts.dtype.is_floating_point:
        # integer runtime scalars: the constant in ``mean``, no draw
        return torch.full(ts.shape, int(ts.mean), dtype=ts.dtype)
    out = torch.empty(n, dtype=ts.dtype)
    # Chunked so that a 235M-element weight does not need a 1 GB fp32 temporary.
    # The stream of normals is the same as one randn(n) call would give.
    off = 0
    while off < n:
        c = min(_CHUNK, n - off)
        v = torch.randn(c, dtype=torch.float32, generator=g)
        out[off:off + c] = (v * ts.std + ts.mean).to(ts.dtype)
        off += c
    return out.view(ts.shape)


def generate(workload: str, dims: Dict[str, int] | None = None,
             seed: int = 0, dtype: torch.dtype | None = None) -> Dict[str, torch.Tensor]:
    """Draw every tensor of ``workload`` (CPU, storage dtype), in order.

    ``dtype`` replaces every tensor's storage dtype (the same normals,
    rounded once to that dtype instead)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    specs = spec(workload, dims)
    if dtype is not None:
        specs = [dataclasses.replace(ts, dtype=dtype) if ts.dtype.is_floating_point else ts
                 for ts in specs]
    return {ts.name: _draw(ts, g) for ts in specs}
