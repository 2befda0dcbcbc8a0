"""Python face of the C ABI: graph builder and compiled plan.

``Graph`` records tensors, step-1 range views and ops ("Implementing a Mega
Kernel for B300", section 1: ops are calls on a graph object, epilogues are
op arguments).  ``Graph.build`` runs the host compiler and returns a
``Plan``; ``Plan.run`` launches the persistent megakernel once per forward
on a torch stream.  PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, byref, c_int32, c_int64, c_void_p
from typing import Dict, List, Optional, Sequence, Union

import numpy as np

from . import _lib as L

_DT = {"f16": L.MK_F16, "bf16": L.MK_BF16, "f32": L.MK_F32, "i32": L.MK_I32}
_ROLE = {"input": L.MK_INPUT, "weight": L.MK_WEIGHT, "output": L.MK_OUTPUT,
         "intermediate": L.MK_INTERMEDIATE}


def _dt(x) -> int:
    if isinstance(x, int):
        return x
    if isinstance(x, str):
        return _DT[x]
    import torch
    return {torch.float16: L.MK_F16, torch.bfloat16: L.MK_BF16, torch.float32: L.MK_F32,
            torch.int32: L.MK_I32}[x]


def _tile(t: Optional[Dict[str, int]]) -> L.Tile:
    tl = L.Tile()
    for k, v in (t or {}).items():
        setattr(tl, k, int(v))
    return tl


class Graph:
    def __init__(self):
        self._lib = L.load()
        self._g = c_void_p()
        L.check(self._lib.mk_graph_create(byref(self._g)))
        self.ids: Dict[str, int] = {}
        self.shapes: Dict[int, tuple] = {}
        self.roles: Dict[int, str] = {}
        self.n_ops = 0

    def __del__(self):
        if getattr(self, "_g", None) and self._g.value:
            self._lib.mk_graph_destroy(self._g)
            self._g = c_void_p()

    # tensors and views -------------------------------------------------
    def tensor(self, name: str, dtype, shape: Sequence[int], role: str) -> int:
        sh = (c_int64 * len(shape))(*shape)
        i = c_int32()
        L.check(self._lib.mk_graph_tensor(self._g, _dt(dtype), len(shape), sh, _ROLE[role],
                                          byref(i)))
        self.ids[name] = i.value
        self.shapes[i.value] = tuple(shape)
        self.roles[i.value] = role
        return i.value

    def view(self, src: int, lo: Sequence[int], hi: Sequence[int]) -> int:
        i = c_int32()
        L.check(self._lib.mk_graph_view(self._g, src, (c_int64 * 4)(*lo), (c_int64 * 4)(*hi),
                                        byref(i)))
        return i.value

    def _padded(self, t: int):
        s = self.shapes[t]
        return (1,) * (4 - len(s)) + tuple(s)

    def cols(self, t: int, c0: int, c1: int) -> int:
        p = self._padded(t)
        return self.view(t, (0, 0, 0, c0), (p[0], p[1], p[2], c1))

    def select0(self, t: int, i: int) -> int:
        p = self._padded(t)
        return self.view(t, (0, i, 0, 0), (1, i + 1, p[2], p[3]))

    # ops ---------------------------------------------------------------
    def _op(self, kind: int, ins: Sequence[int], out: int, attrs: L.OpAttrs) -> None:
        arr = (c_int32 * len(ins))(*ins)
        L.check(self._lib.mk_graph_op(self._g, kind, arr, len(ins), out, byref(attrs)))
        self.n_ops += 1

    def gemm(self, a: int, b: int, out: int, epilogue: int = 0, bias: int = None,
             residual: int = None, gamma: int = None, eps: float = 0.0, head_dim: int = 0,
             rope_cols: int = 0, rope_theta: float = 0.0, tile: Dict[str, int] = None) -> None:
        ins = [a, b]
        if epilogue & L.EP_BIAS:
            ins.append(bias)
        if epilogue & L.EP_RESIDUAL:
            ins.append(residual)
        if epilogue & L.EP_RMSNORM_INPUT:
            ins.append(gamma)
        at = L.OpAttrs(epilogue=epilogue, eps=eps, rope_theta=rope_theta, head_dim=head_dim,
                       rope_cols=rope_cols, tile=_tile(tile))
        self._op(L.MK_OP_GEMM, ins, out, at)

    def rmsnorm(self, x: int, gamma: int, out: int, eps: float = 0.0,
                tile: Dict[str, int] = None) -> None:
        self._op(L.MK_OP_RMSNORM, [x, gamma], out, L.OpAttrs(eps=eps, tile=_tile(tile)))

    def attention(self, q: int, k: int, v: int, out: int, heads: int, kv_heads: int,
                  head_dim: int, causal: bool = True, tile: Dict[str, int] = None) -> None:
        at = L.OpAttrs(n_heads=heads, n_kv_heads=kv_heads, head_dim=head_dim,
                       causal=int(causal), tile=_tile(tile))
        self._op(L.MK_OP_ATTENTION, [q, k, v], out, at)

    def decode_attention(self, q: int, k_new: int, v_new: int, k_cache: int, v_cache: int,
                         pos: int, out: int, heads: int, kv_heads: int, head_dim: int,
                         rope_theta: float = 0.0, tile: Dict[str, int] = None) -> None:
        """Split-KV attention of one new token over a KV cache, with rotary
        embedding at the run-time position ``pos`` and the append of the
        new k, v to the caches (MK_OP_DECODE_ATTENTION in mk.h)."""
        at = L.OpAttrs(n_heads=heads, n_kv_heads=kv_heads, head_dim=head_dim,
                       rope_theta=rope_theta, tile=_tile(tile))
        self._op(L.MK_OP_DECODE_ATTENTION, [q, k_new, v_new, k_cache, v_cache, pos], out, at)

    def add(self, a: int, b: int, out: int, tile: Dict[str, int] = None) -> None:
        self._op(L.MK_OP_ADD, [a, b], out, L.OpAttrs(tile=_tile(tile)))

    def relu(self, a: int, out: int, tile: Dict[str, int] = None) -> None:
        self._op(L.MK_OP_RELU, [a], out, L.OpAttrs(tile=_tile(tile)))

    # compile -----------------------------------------------------------
    def build(self, num_cus: int = 0, cluster_size: int = 0, reuse: int = 0,
              gemv_max_m: int = 0, spin_limit_us: int = 0, cooperative: int = 0,
              pack: int = 0, sync: int = 0, queue: int = 0, debug_poison: int = 0) -> "Plan":
        opts = L.BuildOptions(num_cus=num_cus, cluster_size=cluster_size, reuse=reuse,
                              gemv_max_m=gemv_max_m, spin_limit_us=spin_limit_us,
                              cooperative=cooperative, pack=pack, sync=sync, queue=queue,
                              debug_poison=debug_poison)
        p = c_void_p()
        L.check(self._lib.megakernel_build(self._g, byref(opts), byref(p)))
        return Plan(p, self)


class Plan:
    """A compiled graph.  Owns its device records, counters and intermediates."""

    def __init__(self, handle: c_void_p, graph: Graph):
        self._lib = L.load()
        self._p = handle
        self.ids = dict(graph.ids)
        self.roles = dict(graph.roles)
        self.shapes = dict(graph.shapes)
        self.n_ops = graph.n_ops

    def __del__(self):
        if getattr(self, "_p", None) and self._p.value:
            self._lib.mk_plan_destroy(self._p)
            self._p = c_void_p()

    # introspection -----------------------------------------------------
    def stats(self) -> L.PlanStats:
        s = L.PlanStats()
        L.check(self._lib.mk_plan_stats_get(self._p, byref(s)))
        return s

    def instructions(self) -> np.ndarray:
        w, n, wpi = POINTER(c_int32)(), c_int64(), c_int32()
        L.check(self._lib.mk_plan_instructions(self._p, byref(w), byref(n), byref(wpi)))
        if n.value == 0:
            return np.zeros((0, wpi.value), np.int32)
        return np.ctypeslib.as_array(w, shape=(n.value, wpi.value)).copy()

    def nodes(self) -> np.ndarray:
        w, n, wpn = POINTER(c_int32)(), c_int64(), c_int32()
        L.check(self._lib.mk_plan_nodes(self._p, byref(w), byref(n), byref(wpn)))
        if n.value == 0:
            return np.zeros((0, wpn.value), np.int32)
        return np.ctypeslib.as_array(w, shape=(n.value, wpn.value)).copy()

    def barriers(self) -> np.ndarray:
        w, n = POINTER(c_int32)(), c_int64()
        L.check(self._lib.mk_plan_barriers(self._p, byref(w), byref(n)))
        if n.value == 0:
            return np.zeros(0, np.int32)
        return np.ctypeslib.as_array(w, shape=(n.value,)).copy()

    def slots(self) -> np.ndarray:
        w, n = POINTER(c_int32)(), c_int64()
        L.check(self._lib.mk_plan_slots(self._p, byref(w), byref(n)))
        return np.ctypeslib.as_array(w, shape=(n.value,)).copy()

    def op_tile(self, op: int) -> Dict[str, int]:
        t = L.Tile()
        L.check(self._lib.mk_plan_op_tile(self._p, op, byref(t)))
        return t.as_dict()

    def op_tiles(self) -> List[Dict[str, int]]:
        return [self.op_tile(i) for i in range(self.n_ops)]

    def weight_layout(self, tensor: Union[int, str]):
        """(packed, bytes): whether runs read this weight as packed column
        tiles, and the size of the packed buffer."""
        tid = self.ids[tensor] if isinstance(tensor, str) else tensor
        pk, nb = c_int32(), c_int64()
        L.check(self._lib.mk_plan_weight_layout(self._p, tid, byref(pk), byref(nb)))
        return bool(pk.value), nb.value

    def packed_weights(self) -> List[str]:
        return [n for n, i in self.ids.items()
                if self.roles.get(i) == "weight" and self.weight_layout(i)[0]]

    def pack_weight(self, tensor: Union[int, str], src, dst, stream=None) -> None:
        """Fill device buffer ``dst`` with the packed layout of row-major
        weight ``src`` (both device tensors or pointers)."""
        tid = self.ids[tensor] if isinstance(tensor, str) else tensor
        sp = src if isinstance(src, int) else src.data_ptr()
        dp = dst if isinstance(dst, int) else dst.data_ptr()
        L.check(self._lib.mk_plan_pack_weight(self._p, tid, c_void_p(sp), c_void_p(dp),
                                              self._stream(stream)))

    @property
    def epoch(self) -> int:
        e = c_int64()
        L.check(self._lib.mk_plan_epoch(self._p, byref(e)))
        return e.value

    def decoded(self) -> List[tuple]:
        """Records as (index, cu, iteration, opcode, flags, node, coords,
        ((counter, target), ...), ((counter, arrival rank or -1), ...))."""
        w = self.instructions()
        ncu = self.stats().num_cus
        out = []
        for i, r in enumerate(w):
            ns, nd = int(r[L.W_NSRC]), int(r[L.W_NDST])
            src = tuple((int(r[L.W_SRC_ID + k]), int(r[L.W_SRC_TGT + k])) for k in range(ns))
            dst = tuple((int(r[L.W_DST_ID + k]), int(r[L.W_DST_RANK + k])) for k in range(nd))
            out.append((i, i % ncu, i // ncu, int(r[L.W_OPCODE]), int(r[L.W_FLAGS]),
                        int(r[L.W_NODE]), tuple(int(x) for x in r[L.W_COORD:L.W_COORD + 4]),
                        src, dst))
        return out

    # run ---------------------------------------------------------------
    def _ptrs(self, buffers: Union[Dict[str, "object"], Sequence]) -> ctypes.Array:
        n = max(self.ids.values()) + 1 if self.ids else 0
        n = max(n, L.MAX_TENSORS)
        arr = (c_void_p * n)()
        if isinstance(buffers, dict):
            for name, t in buffers.items():
                arr[self.ids[name]] = t if isinstance(t, int) else t.data_ptr()
        else:
            for i, t in enumerate(buffers):
                if t is not None:
                    arr[i] = t if isinstance(t, int) else t.data_ptr()
        return arr

    @staticmethod
    def _stream(stream) -> c_void_p:
        if stream is None:
            import torch
            stream = torch.cuda.current_stream()
        return c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)

    def run(self, buffers, stream=None) -> None:
        """One forward: one persistent launch of num_cus workgroups on
        ``stream`` (an ordinary launch unless the plan was built with
        ``cooperative=1``; residency as described at megakernel_run)."""
        arr = self._ptrs(buffers)
        L.check(self._lib.megakernel_run(self._p, arr, len(arr), self._stream(stream)))

    def run_traced(self, buffers, trace, stream=None) -> None:
        """One forward that also records 4 wall-clock stamps per instruction
        into ``trace`` (a device int64 tensor of 4 * n_iters * num_cus +
        4 * num_cus; the tail holds per-workgroup clock pairs, see mk.h)."""
        arr = self._ptrs(buffers)
        st = self.stats()
        if trace.numel() < 4 * st.n_iters * st.num_cus + 4 * st.num_cus:
            raise ValueError("trace buffer too small")
        L.check(self._lib.megakernel_run_traced(self._p, arr, len(arr), self._stream(stream),
                                                c_void_p(trace.data_ptr())))

    def run_per_op(self, buffers, stream=None) -> None:
        """Same graph with one launch per node (the per-op baseline)."""
        arr = self._ptrs(buffers)
        L.check(self._lib.megakernel_run_per_op(self._p, arr, len(arr), self._stream(stream)))

    def run_noalloc(self, buffers, stream=None) -> None:
        """One forward through megakernel_run_noalloc: the plan's device
        state in the library's fixed per-GPU array, no allocation."""
        arr = self._ptrs(buffers)
        L.check(self._lib.megakernel_run_noalloc(self._p, arr, len(arr), self._stream(stream)))

    def check(self, stream=None) -> L.RunError:
        """Synchronise and raise MkError(MK_E_DEADLOCK) if a wait gave up."""
        err = L.RunError()
        L.check(self._lib.mk_plan_check(self._p, self._stream(stream), byref(err)))
        return err

    def read_counters(self, stream=None) -> np.ndarray:
        n = len(self.barriers())
        buf = (c_int32 * max(n, 1))()
        L.check(self._lib.mk_plan_read_counters(self._p, buf, max(n, 1), self._stream(stream)))
        return np.array(buf[:n], dtype=np.int64)
