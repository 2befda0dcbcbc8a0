"""The five workload graphs, built through the C ABI.

``build(workload, dims, tiles)`` returns a ``Graph``; ``Runner`` binds
device copies of the seeded inputs, builds the plan and runs forwards.
Weights are K-major ([K, N], y = x @ W).

mlp3        x = relu(x @ W[i] + b[i]) per layer ("MegaKittens Internals",
            section 02); ``fused=False`` gives the nine traced aten ops.
decode      one decoder layer at batch 1: RMSNorm-input QKV GEMV, O + residual,
            RMSNorm-input gate_up with SiLU-mul, down + residual ("Implementing
            a Mega Kernel for B300", sections 1-2).
prefill     Y = X @ W1, Z = relu(Y @ W2) ("Hand-writing a Blackwell GEMM",
            "Two workloads, not one").
decode_gemm Q = X0 @ Wqkv, A = Q[:, :n_q] @ Wo, U = A @ Wup, D = U @ Wdown
            (same page, the M = 256 shapes).
layer       Llama-style decoder layer prefill: RMSNorm, QKV with rotary
            epilogue, causal GQA attention, O + residual, RMSNorm, gate_up
            with SiLU-mul, down + residual ("Beating torch.compile with
            Megakernels in CuTe DSL", "Model Architecture").
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

from . import _lib as L
from .graph import Graph, Plan

OUTPUT = dict(mlp3=None, decode="out", prefill="Z", decode_gemm="D", layer="out", decode_kv="out")
DTYPE = dict(mlp3="f16", decode="bf16", prefill="f16", decode_gemm="f16", layer="bf16",
             decode_kv="bf16")


def output_name(workload: str, dims: Dict[str, int]) -> str:
    if workload == "mlp3":
        return f"y{dims['layers'] - 1}"
    return OUTPUT[workload]


def _t(tiles, i):
    if not tiles:
        return None
    return tiles[i] if i < len(tiles) else None


def build(workload: str, dims: Dict[str, int], tiles: Optional[Sequence[dict]] = None,
          fused: bool = True, w_first: bool = False, dtype: Optional[str] = None) -> Graph:
    """``dtype`` overrides mlp3's fp16 (the traced MLP of MegaKittens
    Internals, section 02, is bf16)."""
    g = Graph()
    d = dims
    if workload == "mlp3":
        Lh, M, H = d["layers"], d["m"], d["h"]
        dt = dtype or "f16"
        if w_first:
            W = g.tensor("W", dt, (Lh, H, H), "weight")
            x = g.tensor("x", dt, (M, H), "input")
            b = g.tensor("b", dt, (Lh, M, H), "weight")
        else:
            x = g.tensor("x", dt, (M, H), "input")
            W = g.tensor("W", dt, (Lh, H, H), "weight")
            b = g.tensor("b", dt, (Lh, M, H), "weight")
        cur = x
        for i in range(Lh):
            last = i == Lh - 1
            if fused:
                y = g.tensor(f"y{i}", dt, (M, H), "output" if last else "intermediate")
                g.gemm(cur, g.select0(W, i), y, L.EP_BIAS | L.EP_RELU, bias=g.select0(b, i),
                       tile=_t(tiles, i) if tiles and len(tiles) > 1 else _t(tiles, 0))
                cur = y
            else:
                mm = g.tensor(f"mm{i}", dt, (M, H), "intermediate")
                g.gemm(cur, g.select0(W, i), mm, 0, tile=tiles[0]["gemm"] if tiles else None)
                ad = g.tensor(f"add{i}", dt, (M, H), "intermediate")
                g.add(mm, g.select0(b, i), ad, tile=tiles[0]["ew"] if tiles else None)
                r = g.tensor(f"relu{i}" if not last else f"y{i}", dt, (M, H),
                             "output" if last else "intermediate")
                g.relu(ad, r, tile=tiles[0]["ew"] if tiles else None)
                cur = r
        return g
    if workload == "prefill":
        X = g.tensor("X", "f16", (d["m"], d["k"]), "input")
        W1 = g.tensor("W1", "f16", (d["k"], d["n1"]), "weight")
        W2 = g.tensor("W2", "f16", (d["n1"], d["n2"]), "weight")
        Y = g.tensor("Y", "f16", (d["m"], d["n1"]), "intermediate")
        Z = g.tensor("Z", "f16", (d["m"], d["n2"]), "output")
        g.gemm(X, W1, Y, 0, tile=_t(tiles, 0))
        g.gemm(Y, W2, Z, L.EP_RELU, tile=_t(tiles, 1))
        return g
    if workload == "decode_gemm":
        M, K = d["m"], d["k"]
        X0 = g.tensor("X0", "f16", (M, K), "input")
        Wqkv = g.tensor("Wqkv", "f16", (K, d["n_qkv"]), "weight")
        Wo = g.tensor("Wo", "f16", (d["n_q"], d["n_o"]), "weight")
        Wup = g.tensor("Wup", "f16", (d["n_o"], d["n_up"]), "weight")
        Wdn = g.tensor("Wdown", "f16", (d["n_up"], d["n_down"]), "weight")
        Q = g.tensor("Q", "f16", (M, d["n_qkv"]), "intermediate")
        A = g.tensor("A", "f16", (M, d["n_o"]), "intermediate")
        U = g.tensor("U", "f16", (M, d["n_up"]), "intermediate")
        D = g.tensor("D", "f16", (M, d["n_down"]), "output")
        g.gemm(X0, Wqkv, Q, 0, tile=_t(tiles, 0))
        g.gemm(g.cols(Q, 0, d["n_q"]), Wo, A, 0, tile=_t(tiles, 1))
        g.gemm(A, Wup, U, 0, tile=_t(tiles, 2))
        g.gemm(U, Wdn, D, 0, tile=_t(tiles, 3))
        return g
    if workload == "decode":
        M, H, nq, I = d["m"], d["hidden"], d["n_q"], d["inter"]
        nqkv = nq + 2 * d["n_kv"]
        x = g.tensor("x", "bf16", (M, H), "input")
        g1 = g.tensor("g1", "bf16", (H,), "weight")
        Wqkv = g.tensor("Wqkv", "bf16", (H, nqkv), "weight")
        Wo = g.tensor("Wo", "bf16", (nq, H), "weight")
        g2 = g.tensor("g2", "bf16", (H,), "weight")
        Wgu = g.tensor("Wgu", "bf16", (H, 2 * I), "weight")
        Wd = g.tensor("Wd", "bf16", (I, H), "weight")
        qkv = g.tensor("qkv", "bf16", (M, nqkv), "intermediate")
        h = g.tensor("h", "bf16", (M, H), "intermediate")
        a = g.tensor("a", "bf16", (M, I), "intermediate")
        out = g.tensor("out", "bf16", (M, H), "output")
        g.gemm(x, Wqkv, qkv, L.EP_RMSNORM_INPUT, gamma=g1, tile=_t(tiles, 0))
        g.gemm(g.cols(qkv, 0, nq), Wo, h, L.EP_RESIDUAL, residual=x, tile=_t(tiles, 1))
        g.gemm(h, Wgu, a, L.EP_RMSNORM_INPUT | L.EP_SILU_MUL, gamma=g2, tile=_t(tiles, 2))
        g.gemm(a, Wd, out, L.EP_RESIDUAL, residual=h, tile=_t(tiles, 3))
        return g
    if workload == "decode_kv":
        # the decode layer with its attention: rotary q, k at the run-time
        # position, split-KV attention over the cache with the append of
        # the new k, v, then O + residual and the MLP as in ``decode``
        M, H, nq, nkv, I, hd = d["m"], d["hidden"], d["n_q"], d["n_kv"], d["inter"], d["head_dim"]
        Smax = d["s_max"]
        x = g.tensor("x", "bf16", (M, H), "input")
        g1 = g.tensor("g1", "bf16", (H,), "weight")
        Wqkv = g.tensor("Wqkv", "bf16", (H, nq + 2 * nkv), "weight")
        Wo = g.tensor("Wo", "bf16", (nq, H), "weight")
        g2 = g.tensor("g2", "bf16", (H,), "weight")
        Wgu = g.tensor("Wgu", "bf16", (H, 2 * I), "weight")
        Wd = g.tensor("Wd", "bf16", (I, H), "weight")
        kc = g.tensor("k_cache", "bf16", (Smax, nkv), "input")
        vc = g.tensor("v_cache", "bf16", (Smax, nkv), "input")
        pos = g.tensor("pos", "i32", (1,), "input")
        qkv = g.tensor("qkv", "bf16", (M, nq + 2 * nkv), "intermediate")
        o = g.tensor("o", "bf16", (M, nq), "intermediate")
        h = g.tensor("h", "bf16", (M, H), "intermediate")
        a = g.tensor("a", "bf16", (M, I), "intermediate")
        out = g.tensor("out", "bf16", (M, H), "output")
        g.gemm(x, Wqkv, qkv, L.EP_RMSNORM_INPUT, gamma=g1, tile=_t(tiles, 0))
        g.decode_attention(g.cols(qkv, 0, nq), g.cols(qkv, nq, nq + nkv), g.cols(qkv, nq + nkv, nq + 2 * nkv),
                           kc, vc, pos, o, nq // hd, nkv // hd, hd, tile=_t(tiles, 1))
        g.gemm(o, Wo, h, L.EP_RESIDUAL, residual=x, tile=_t(tiles, 2))
        g.gemm(h, Wgu, a, L.EP_RMSNORM_INPUT | L.EP_SILU_MUL, gamma=g2, tile=_t(tiles, 3))
        g.gemm(a, Wd, out, L.EP_RESIDUAL, residual=h, tile=_t(tiles, 4))
        return g
    if workload == "layer":
        S, H = d["seq"], d["hidden"]
        Hq, Hkv, hd, I = d["heads"], d["kv_heads"], d["head_dim"], d["inter"]
        nq, nkv = Hq * hd, Hkv * hd
        x = g.tensor("x", "bf16", (S, H), "input")
        g1 = g.tensor("g1", "bf16", (H,), "weight")
        # Wqkv = [Wq | Wkv], held as two weights so that each projection
        # reads a whole weight and takes the packed GEMM body
        Wq = g.tensor("Wq", "bf16", (H, nq), "weight")
        Wkv = g.tensor("Wkv", "bf16", (H, 2 * nkv), "weight")
        Wo = g.tensor("Wo", "bf16", (nq, H), "weight")
        g2 = g.tensor("g2", "bf16", (H,), "weight")
        Wgu = g.tensor("Wgu", "bf16", (H, 2 * I), "weight")
        Wd = g.tensor("Wd", "bf16", (I, H), "weight")
        xn = g.tensor("xn", "bf16", (S, H), "intermediate")
        q = g.tensor("q", "bf16", (S, nq), "intermediate")
        kv = g.tensor("kv", "bf16", (S, 2 * nkv), "intermediate")
        o = g.tensor("o", "bf16", (S, nq), "intermediate")
        h1 = g.tensor("h1", "bf16", (S, H), "intermediate")
        hn = g.tensor("hn", "bf16", (S, H), "intermediate")
        a = g.tensor("a", "bf16", (S, I), "intermediate")
        out = g.tensor("out", "bf16", (S, H), "output")
        # The QKV projection runs as two GEMMs (q, and k|v): each attention
        # instruction then depends on one q tile set per head and one k|v set
        # per kv head instead of a unique union.
        g.rmsnorm(x, g1, xn, tile=_t(tiles, 0))
        g.gemm(xn, Wq, q, L.EP_ROPE, head_dim=hd, rope_cols=nq, tile=_t(tiles, 1))
        g.gemm(xn, Wkv, kv, L.EP_ROPE, head_dim=hd, rope_cols=nkv, tile=_t(tiles, 2))
        g.attention(q, g.cols(kv, 0, nkv), g.cols(kv, nkv, 2 * nkv), o, Hq, Hkv, hd, True,
                    tile=_t(tiles, 3))
        g.gemm(o, Wo, h1, L.EP_RESIDUAL, residual=x, tile=_t(tiles, 4))
        g.rmsnorm(h1, g2, hn, tile=_t(tiles, 5))
        g.gemm(hn, Wgu, a, L.EP_SILU_MUL, tile=_t(tiles, 6))
        g.gemm(a, Wd, out, L.EP_RESIDUAL, residual=h1, tile=_t(tiles, 7))
        return g
    raise KeyError(workload)


def layer_stack(dims: Dict[str, int], n_layers: int, tiles: Optional[Sequence[dict]] = None) -> Graph:
    """``n_layers`` of the prefill decoder layer in sequence (the layer
    graph above, each with its own weights): tensors ``x``, per layer l the
    weights ``g1_l, Wq_l, Wkv_l, Wo_l, g2_l, Wgu_l, Wd_l`` and the layer's
    output ``out_l`` (the graph output for the last layer), which is the next
    layer's input."""
    g = Graph()
    S, H = dims["seq"], dims["hidden"]
    Hq, Hkv, hd, I = dims["heads"], dims["kv_heads"], dims["head_dim"], dims["inter"]
    nq, nkv = Hq * hd, Hkv * hd
    cur = g.tensor("x", "bf16", (S, H), "input")
    for l in range(n_layers):
        g1 = g.tensor(f"g1_{l}", "bf16", (H,), "weight")
        Wq = g.tensor(f"Wq_{l}", "bf16", (H, nq), "weight")
        Wkv = g.tensor(f"Wkv_{l}", "bf16", (H, 2 * nkv), "weight")
        Wo = g.tensor(f"Wo_{l}", "bf16", (nq, H), "weight")
        g2 = g.tensor(f"g2_{l}", "bf16", (H,), "weight")
        Wgu = g.tensor(f"Wgu_{l}", "bf16", (H, 2 * I), "weight")
        Wd = g.tensor(f"Wd_{l}", "bf16", (I, H), "weight")
        xn = g.tensor(f"xn_{l}", "bf16", (S, H), "intermediate")
        q = g.tensor(f"q_{l}", "bf16", (S, nq), "intermediate")
        kv = g.tensor(f"kv_{l}", "bf16", (S, 2 * nkv), "intermediate")
        o = g.tensor(f"o_{l}", "bf16", (S, nq), "intermediate")
        h1 = g.tensor(f"h1_{l}", "bf16", (S, H), "intermediate")
        hn = g.tensor(f"hn_{l}", "bf16", (S, H), "intermediate")
        a = g.tensor(f"a_{l}", "bf16", (S, I), "intermediate")
        out = g.tensor(f"out_{l}", "bf16", (S, H), "output" if l == n_layers - 1 else "intermediate")
        g.rmsnorm(cur, g1, xn, tile=_t(tiles, 0))
        g.gemm(xn, Wq, q, L.EP_ROPE, head_dim=hd, rope_cols=nq, tile=_t(tiles, 1))
        g.gemm(xn, Wkv, kv, L.EP_ROPE, head_dim=hd, rope_cols=nkv, tile=_t(tiles, 2))
        g.attention(q, g.cols(kv, 0, nkv), g.cols(kv, nkv, 2 * nkv), o, Hq, Hkv, hd, True,
                    tile=_t(tiles, 3))
        g.gemm(o, Wo, h1, L.EP_RESIDUAL, residual=cur, tile=_t(tiles, 4))
        g.rmsnorm(h1, g2, hn, tile=_t(tiles, 5))
        g.gemm(hn, Wgu, a, L.EP_SILU_MUL, tile=_t(tiles, 6))
        g.gemm(a, Wd, out, L.EP_RESIDUAL, residual=h1, tile=_t(tiles, 7))
        cur = out
    return g


def graph_inputs(workload: str, dims: Dict[str, int], inputs: Dict[str, "object"]) -> Dict[str, "object"]:
    """The graph's input and weight tensors from a workload's inputs: the
    layer's Wqkv is handed over as its q and k|v column blocks."""
    out = dict(inputs)
    if workload == "layer" and "Wqkv" in out:
        nq = dims["heads"] * dims["head_dim"]
        w = out.pop("Wqkv")
        out["Wq"] = w[:, :nq].contiguous()
        out["Wkv"] = w[:, nq:].contiguous()
    return out


class Runner:
    """Device copies of a workload's inputs, its plan, and forwards."""

    def __init__(self, workload: str, dims: Dict[str, int], inputs: Dict[str, "object"],
                 tiles: Optional[Sequence[dict]] = None, device: str = "cuda", **opts):
        import torch
        self.workload, self.dims = workload, dims
        self.graph = build(workload, dims, tiles)
        self.plan: Plan = self.graph.build(**opts)
        self.bufs = {k: v.to(device).contiguous() for k, v in graph_inputs(workload, dims, inputs).items()}
        # weights the plan reads as packed column tiles: pack once, run on the copy
        self.packed = {}
        for name in self.plan.packed_weights():
            nbytes = self.plan.weight_layout(name)[1]
            dst = torch.empty(nbytes // 2, dtype=self.bufs[name].dtype, device=device)
            self.plan.pack_weight(name, self.bufs[name], dst)
            self.packed[name] = dst
        self.run_bufs = dict(self.bufs)
        self.run_bufs.update(self.packed)
        self.out_name = output_name(workload, dims)
        oid = self.graph.ids[self.out_name]
        tdt = torch.float16 if DTYPE[workload] == "f16" else torch.bfloat16
        self.out = torch.empty(self.graph.shapes[oid], dtype=tdt, device=device)
        self.bufs[self.out_name] = self.out
        self.run_bufs[self.out_name] = self.out

    def alt_plan(self, **opts) -> Plan:
        """Another plan of the same graph (e.g. ``queue=1``); it must read
        its weights in the same layouts, so it runs on this runner's
        buffers."""
        p = self.graph.build(**opts)
        if sorted(p.packed_weights()) != sorted(self.packed):
            raise ValueError("alternative plan packs other weights")
        for name, buf in self.packed.items():
            if p.weight_layout(name)[1] != buf.numel() * buf.element_size():
                raise ValueError(f"alternative plan packs {name} in another layout")
        return p

    def forward(self, stream=None, plan: Optional[Plan] = None):
        (plan or self.plan).run(self.run_bufs, stream)
        return self.out

    def forward_per_op(self, stream=None):
        self.plan.run_per_op(self.run_bufs, stream)
        return self.out
