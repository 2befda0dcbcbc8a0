"""ctypes binding of libmk.so (the C ABI declared in include/mk.h).

Argument marshalling only: every step of the compile and of the forward runs
inside the shared library.  Loading fails loudly when the library has not
been built (``python -m tiled_gemm_graph_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, byref, c_char_p, c_double, c_float, c_int, c_int32, \
    c_int64, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmk.so")

MK_OK, MK_E_INVALID, MK_E_UNSUPPORTED, MK_E_LIMIT, MK_E_HIP, MK_E_DEADLOCK = range(6)
STATUS_NAMES = ["MK_OK", "MK_E_INVALID", "MK_E_UNSUPPORTED", "MK_E_LIMIT", "MK_E_HIP",
                "MK_E_DEADLOCK"]
MK_F16, MK_BF16, MK_F32, MK_I32 = 1, 2, 3, 4
MK_INPUT, MK_WEIGHT, MK_OUTPUT, MK_INTERMEDIATE = 0, 1, 2, 3
MK_OP_GEMM, MK_OP_RMSNORM, MK_OP_ATTENTION, MK_OP_ADD, MK_OP_RELU, MK_OP_DECODE_ATTENTION = (
    1, 2, 3, 4, 5, 6)
EP_BIAS, EP_RELU, EP_RESIDUAL, EP_SILU_MUL, EP_RMSNORM_INPUT, EP_ROPE, EP_PARTIAL = (
    1, 2, 4, 8, 16, 32, 64)
(I_NOOP, I_GEMM, I_GEMV, I_REDUCE, I_RMSNORM, I_ATTENTION, I_EW_ADD, I_EW_RELU, I_ATTN_PARTIAL,
 I_ATTN_COMBINE) = range(10)
MAX_TENSORS, MAX_SRC, MAX_DST, INSTR_WORDS, NODE_WORDS = 256, 16, 8, 64, 64

# word offsets of mk_instr (mirrors the struct; checked by tests)
W_OPCODE, W_FLAGS, W_NODE, W_NSRC, W_NDST = 0, 1, 2, 3, 4
W_COORD = 5
W_R0, W_R1, W_C0, W_C1, W_K0, W_K1, W_SPLIT = 9, 10, 11, 12, 13, 14, 15
W_SRC_ID = 16
W_SRC_TGT = W_SRC_ID + MAX_SRC
W_DST_ID = W_SRC_TGT + MAX_SRC
W_DST_RANK = W_DST_ID + MAX_DST
# node descriptor words (mk_node)
N_LAYOUT, N_LINES_OWN = 56, 57
SLICE_MAX = 256  # counters with at most this target are one slot per arrival


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 6 else status}: {msg}")
        self.status = status


class Tile(Structure):
    _fields_ = [(n, c_int32) for n in
                ("bm", "bn", "split", "dup", "gemv", "rbm", "rbn", "rows", "bq", "er", "ec",
                 "layout")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class OpAttrs(Structure):
    _fields_ = [("epilogue", c_uint32), ("eps", c_float), ("rope_theta", c_float),
                ("n_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("causal", c_int32), ("rope_cols", c_int32), ("tile", Tile)]


class BuildOptions(Structure):
    _fields_ = [("num_cus", c_int32), ("cluster_size", c_int32), ("reuse", c_int32),
                ("gemv_max_m", c_int32), ("spin_limit_us", c_int64),
                ("cooperative", c_int32), ("pack", c_int32), ("sync", c_int32),
                ("queue", c_int32), ("debug_poison", c_int32)]


class PlanStats(Structure):
    _fields_ = [("n_instr", c_int64), ("n_iters", c_int64), ("n_nodes", c_int64),
                ("n_barriers", c_int64), ("n_input_barriers", c_int64),
                ("n_reuse_barriers", c_int64), ("n_slots", c_int64),
                ("intermediate_bytes", c_int64), ("flops", c_double), ("bytes", c_double),
                ("num_cus", c_int32), ("reserved", c_int32)]


class RunError(Structure):
    _fields_ = [(n, c_int32) for n in ("code", "cu", "instr", "barrier", "value", "need")]


EXPORTS = [
    "mk_graph_create", "mk_graph_destroy", "mk_graph_tensor", "mk_graph_view", "mk_graph_op",
    "megakernel_build", "mk_plan_destroy", "megakernel_run", "megakernel_run_traced",
    "megakernel_run_per_op", "megakernel_run_noalloc",
    "mk_plan_check", "mk_plan_stats_get", "mk_plan_instructions", "mk_plan_nodes",
    "mk_plan_barriers", "mk_plan_slots", "mk_plan_op_tile", "mk_plan_read_counters",
    "mk_plan_epoch", "mk_plan_weight_layout", "mk_plan_pack_weight", "mk_wall_clock_khz",
    "mk_probe_mfma",
    "mk_last_error", "mk_abi_version",
]

_lib = None


def load() -> ctypes.CDLL:
    """Load libmk.so once; raise ImportError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m tiled_gemm_graph_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32p, i64p = c_void_p, POINTER(c_int32), POINTER(c_int64)
    sig = {
        "mk_graph_create": ([POINTER(c_void_p)], c_int),
        "mk_graph_destroy": ([vp], None),
        "mk_graph_tensor": ([vp, c_int, c_int, i64p, c_int, i32p], c_int),
        "mk_graph_view": ([vp, c_int32, i64p, i64p, i32p], c_int),
        "mk_graph_op": ([vp, c_int, i32p, c_int, c_int32, POINTER(OpAttrs)], c_int),
        "megakernel_build": ([vp, POINTER(BuildOptions), POINTER(c_void_p)], c_int),
        "mk_plan_destroy": ([vp], None),
        "megakernel_run": ([vp, POINTER(c_void_p), c_int, vp], c_int),
        "megakernel_run_traced": ([vp, POINTER(c_void_p), c_int, vp, vp], c_int),
        "megakernel_run_per_op": ([vp, POINTER(c_void_p), c_int, vp], c_int),
        "megakernel_run_noalloc": ([vp, POINTER(c_void_p), c_int, vp], c_int),
        "mk_plan_check": ([vp, vp, POINTER(RunError)], c_int),
        "mk_plan_stats_get": ([vp, POINTER(PlanStats)], c_int),
        "mk_plan_instructions": ([vp, POINTER(i32p), i64p, i32p], c_int),
        "mk_plan_nodes": ([vp, POINTER(i32p), i64p, i32p], c_int),
        "mk_plan_barriers": ([vp, POINTER(i32p), i64p], c_int),
        "mk_plan_slots": ([vp, POINTER(i32p), i64p], c_int),
        "mk_plan_op_tile": ([vp, c_int32, POINTER(Tile)], c_int),
        "mk_plan_read_counters": ([vp, i32p, c_int64, vp], c_int),
        "mk_plan_epoch": ([vp, i64p], c_int),
        "mk_plan_weight_layout": ([vp, c_int32, i32p, i64p], c_int),
        "mk_plan_pack_weight": ([vp, c_int32, vp, vp, vp], c_int),
        "mk_wall_clock_khz": ([i32p], c_int),
        "mk_probe_mfma": ([vp, vp, c_int32, c_int32, c_int32, vp], c_int),
        "mk_last_error": ([], c_char_p),
        "mk_abi_version": ([], c_int32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    if L.mk_abi_version() != 5:
        raise ImportError("libmk.so ABI version mismatch")
    _lib = L
    return L


def check(status: int) -> None:
    if status != MK_OK:
        raise MkError(status, load().mk_last_error().decode())
