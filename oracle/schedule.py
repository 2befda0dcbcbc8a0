"""Brute-force oracle of the instruction list, tensor slots and counters.

Test infrastructure only (see the package docstring).

Given a graph (tensors, ops with tile parameters), this module re-derives
what the host compiler must emit, following MegaKittens Internals:

* section 04, phase 1 (count and place): each lowered node gets a
  contiguous range of the flat list in topological order, rounded up to a
  multiple of ``cluster_size`` with Noop pads;
* section 04, phase 2 (tensor slots): graph inputs first, then node outputs
  in node order; a new output may take a pooled slot of identical meta only
  when its node starts at least ``ncu`` instructions after the exclusive end
  of every reader of the slot's previous tensor (reading:
  ``start - end_exclusive >= ncu``);
* section 04, phase 3 (barriers): one counter per distinct (producer node,
  dependency set); target = size of the set; one reuse counter per reuse
  event that every instruction of every old reader arrives on;
* section 05 (placement): instruction i runs on CU i % ncu in iteration
  i // ncu.

Dependency sets here come from testing every consumer read box against
every producer write box (brute force).  The compiler uses the unit-cell
(GCD) method of section 04 instead; equality of the two is the check.

Lowering and tiling spec (the compiler implements the same rules):

``gemm`` op, tile params bm, bn, split S, dup, gemv, rbm, rbn:
  out [M, N]; A view [M, K]; B view [K, Nb] with Nb = 2N under SILU_MUL
  (gate columns first) else N.  K is cut into S chunks of
  Kc = roundup(ceil(K/S), 64) rows (every chunk must be non-empty).
  Tiles run in groups, chunk index s fastest, each tile repeated ``dup``
  times (the CTA-pair duplicate of section 04).  GEMM-body nodes cut the
  TM x TN tile grid into groups of gm = min(TM, 32) rows by
  gn = min(TN, max(1, B // (gm * S))) columns, B = ncu // 8 when ncu is a
  multiple of 8, else 32; groups are taken row by row and the tiles of a
  group row by row.  GEMV-body
  nodes run row-major over (tm, tn).  Placement: a GEMM-body node with at
  least ncu instructions starts on a multiple of ncu // 8 (when ncu is a
  multiple of 8), the gap before it being Noops.
  S == 1: one node (opcode GEMV if gemv else GEMM) with the op's flags.
  S > 1: a partial node (opcode GEMV/GEMM, flags PARTIAL | the op's
  SILU_MUL and RMSNORM_INPUT bits) writing fp32 partials P [S, M, Nb],
  then a REDUCE node over (rbm x rbn) output tiles carrying the op's other
  flags.  Read boxes: A rows x [k0, k1); B [k0, k1) x cols (and x (N+cols)
  under SILU_MUL); gamma [k0, k1) under RMSNORM_INPUT; bias / residual
  rows x cols (S == 1 only).  REDUCE reads P [0, S) x rows x cols (and N +
  cols), bias / residual rows x cols, and under RMSNORM_INPUT the A rows
  over the full K (for the row's sum of squares).
  gemv == 1 with layout == 2 (packed column tiles): one GEMV node, no
  split, no REDUCE;
  tiles (tm, tn) row-major over bm rows x bn output *positions*; each
  instruction covers the whole K.  Position p is output column p, except
  under ROPE for p < rope_cols (default N), where p of head h = p // hd,
  i = (p % hd) // 2 is column h * hd + i + (p % 2) * hd / 2 (the two
  columns of a rotation pair are neighbours in position order).  Reads: A
  rows x [0, K); B [0, K) x the tile's columns (and x N + those columns
  under SILU_MUL); gamma [0, K); bias / residual rows x the columns; writes
  out rows x the columns.
``rmsnorm`` op, tile param rows R: row blocks of R rows; reads x rows x all
  columns and gamma; writes rows x all columns.
``attention`` op, tile param bq: q blocks of bq rows; order: q block
  descending (longest first), head ascending; reads q rows [q0,q1) x head
  columns and k, v rows [0, S) x the kv head's columns (kv head =
  h // (Hq/Hkv)); writes o rows [q0,q1) x head columns.  The k/v boxes cover
  the whole sequence even under the causal mask, so every q block of a kv
  head shares one dependency set and each k/v tile arrives on one counter.
``add`` / ``relu`` ops, tile params er, ec: row-major (er x ec) tiles.
``decode_attention`` op (one new token over a KV cache, "Implementing a
  Mega Kernel for B300", section 2), tile param bq = C keys per chunk:
  partial fp32 tensor P [1, NC, Hq, d + 4] (NC = ceil(S_max / C)) appended
  to the graph; a partial node of NC x Hkv instructions, chunk c outer, kv
  head g inner, coords (c, g), each reading the q columns of g's G = Hq /
  Hkv query heads, k_new and v_new of g, cache rows [cC, min(S, cC + C)) x
  g's columns of both caches, and the position; writing P (chunk c, heads
  of g, all d + 4).  Then a combine node of Hkv instructions, coords (g),
  reading P (all chunks, heads of g) and the position, writing o's columns
  of g's query heads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# opcodes
NOOP, GEMM, GEMV, REDUCE, RMSNORM, ATTENTION, EW_ADD, EW_RELU, ATTN_PARTIAL, ATTN_COMBINE = range(10)
OPCODE_NAMES = ["NOOP", "GEMM", "GEMV", "REDUCE", "RMSNORM", "ATTENTION",
                "EW_ADD", "EW_RELU", "ATTN_PARTIAL", "ATTN_COMBINE"]
# epilogue / role flags
BIAS, RELU, RESIDUAL, SILU_MUL, RMSNORM_INPUT, ROPE, PARTIAL = (
    1, 2, 4, 8, 16, 32, 64)

MAX_SRC, MAX_DST = 16, 8
# Counters with at most this many arrivals are kept as one slot per arrival
# (this library's encoding of a counter in device memory, not a step of the
# method): each arriving instruction then carries its rank, its position
# among the counter's arrivals in instruction order; larger counters carry
# rank -1.
SLICE_MAX = 256
DTYPE_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "i32": 4}


@dataclasses.dataclass
class Tensor:
    name: str
    dtype: str
    shape: Tuple[int, ...]
    role: str  # "input" | "weight" | "output" | "intermediate"

    @property
    def padded(self) -> Tuple[int, int, int, int]:
        s = tuple(self.shape)
        return (1,) * (4 - len(s)) + s


@dataclasses.dataclass
class Edge:
    """A step-1 range on a tensor, in its left-padded 4-D coordinates."""
    tensor: int
    lo: Tuple[int, int, int, int]
    hi: Tuple[int, int, int, int]

    @property
    def rows(self) -> int:
        return self.hi[2] - self.lo[2]

    @property
    def cols(self) -> int:
        return self.hi[3] - self.lo[3]

    def box(self, r0: int, r1: int, c0: int, c1: int):
        """Box on the source tensor for logical rows [r0,r1) x cols [c0,c1)
        of this 2-D view (dims 0 and 1 must have extent 1)."""
        assert self.hi[0] - self.lo[0] == 1 and self.hi[1] - self.lo[1] == 1
        assert 0 <= r0 <= r1 <= self.rows and 0 <= c0 <= c1 <= self.cols
        return ((self.lo[0], self.hi[0]), (self.lo[1], self.hi[1]),
                (self.lo[2] + r0, self.lo[2] + r1),
                (self.lo[3] + c0, self.lo[3] + c1))


@dataclasses.dataclass
class Op:
    kind: str                     # gemm | rmsnorm | attention | add | relu
    ins: Dict[str, Edge]
    out: int
    flags: int = 0
    tile: Dict[str, int] = dataclasses.field(default_factory=dict)
    attrs: Dict[str, float] = dataclasses.field(default_factory=dict)


@dataclasses.dataclass
class Graph:
    tensors: List[Tensor] = dataclasses.field(default_factory=list)
    ops: List[Op] = dataclasses.field(default_factory=list)

    def tensor(self, name, dtype, shape, role) -> int:
        self.tensors.append(Tensor(name, dtype, tuple(shape), role))
        return len(self.tensors) - 1

    def full(self, t: int) -> Edge:
        p = self.tensors[t].padded
        return Edge(t, (0, 0, 0, 0), p)

    def cols(self, t: int, c0: int, c1: int) -> Edge:
        p = self.tensors[t].padded
        return Edge(t, (0, 0, 0, c0), (p[0], p[1], p[2], c1))

    def select0(self, t: int, i: int) -> Edge:
        """t[i] for a 3-D tensor: the (1, i, :, :) slice."""
        p = self.tensors[t].padded
        return Edge(t, (0, i, 0, 0), (1, i + 1, p[2], p[3]))


@dataclasses.dataclass
class Instr:
    coords: Tuple[int, int, int, int]
    reads: List[Tuple[int, tuple]]   # (tensor, box)
    writes: List[Tuple[int, tuple]]


@dataclasses.dataclass
class Node:
    op: int
    opcode: int
    flags: int
    out: int
    edges: List[Edge]
    instrs: List[Instr]
    start: int = 0
    end: int = 0   # exclusive, after padding


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _chunks(K: int, S: int) -> List[Tuple[int, int]]:
    kc = _cdiv(_cdiv(K, S), 64) * 64
    ch = [(s * kc, min(K, (s + 1) * kc)) for s in range(S)]
    if any(k0 >= k1 for k0, k1 in ch):
        raise ValueError(f"split {S} leaves an empty K chunk (K={K})")
    return ch


def lower(g: Graph, ncu: int = 256) -> List[Node]:
    """Lower graph ops to nodes with their instruction boxes (tiling spec in
    the module docstring).  May append partial-sum tensors to ``g``."""
    nodes: List[Node] = []
    for oi, op in enumerate(g.ops):
        if op.kind == "gemm":
            nodes.extend(_lower_gemm(g, oi, op, ncu))
        elif op.kind == "rmsnorm":
            x, gm = op.ins["x"], op.ins["gamma"]
            M, H = x.rows, x.cols
            R = op.tile["rows"]
            ins = []
            for rb in range(_cdiv(M, R)):
                r0, r1 = rb * R, min(M, rb * R + R)
                ins.append(Instr((rb, 0, 0, 0),
                                 [(x.tensor, x.box(r0, r1, 0, H)),
                                  (gm.tensor, gm.box(0, 1, 0, H))],
                                 [(op.out, g.full(op.out).box(r0, r1, 0, H))]))
            nodes.append(Node(oi, RMSNORM, 0, op.out, [x, gm], ins))
        elif op.kind == "attention":
            q, k, v = op.ins["q"], op.ins["k"], op.ins["v"]
            Hq, Hkv = int(op.attrs["heads"]), int(op.attrs["kv_heads"])
            d = int(op.attrs["head_dim"])
            S = q.rows
            bq = op.tile["bq"]
            o = g.full(op.out)
            ins = []
            for qb in reversed(range(_cdiv(S, bq))):
                q0, q1 = qb * bq, min(S, qb * bq + bq)
                kend = S
                for h in range(Hq):
                    kh = h // (Hq // Hkv)
                    ins.append(Instr((qb, h, 0, 0),
                                     [(q.tensor, q.box(q0, q1, h * d, h * d + d)),
                                      (k.tensor, k.box(0, kend, kh * d, kh * d + d)),
                                      (v.tensor, v.box(0, kend, kh * d, kh * d + d))],
                                     [(op.out, o.box(q0, q1, h * d, h * d + d))]))
            # instruction j shares its CU with j + ncu: reverse every other
            # run of ncu (most keys first, then fewest first) so each CU's
            # causal work evens out
            for c0 in range(ncu, len(ins), 2 * ncu):
                ins[c0:c0 + ncu] = ins[c0:c0 + ncu][::-1]
            nodes.append(Node(oi, ATTENTION, 0, op.out, [q, k, v], ins))
        elif op.kind == "decode_attention":
            nodes.extend(_lower_decode_attention(g, oi, op))
        elif op.kind in ("add", "relu"):
            a = op.ins["a"]
            M, N = a.rows, a.cols
            er, ec = op.tile["er"], op.tile["ec"]
            srcs = [a] + ([op.ins["b"]] if op.kind == "add" else [])
            o = g.full(op.out)
            ins = []
            for tr in range(_cdiv(M, er)):
                for tc in range(_cdiv(N, ec)):
                    r0, r1 = tr * er, min(M, tr * er + er)
                    c0, c1 = tc * ec, min(N, tc * ec + ec)
                    ins.append(Instr((tr, tc, 0, 0),
                                     [(e.tensor, e.box(r0, r1, c0, c1)) for e in srcs],
                                     [(op.out, o.box(r0, r1, c0, c1))]))
            nodes.append(Node(oi, EW_ADD if op.kind == "add" else EW_RELU, 0,
                              op.out, srcs, ins))
        else:
            raise ValueError(op.kind)
    return nodes


def _lower_decode_attention(g: Graph, oi: int, op: Op) -> List[Node]:
    q, kn, vn = op.ins["q"], op.ins["k_new"], op.ins["v_new"]
    kc, vc, ps = op.ins["k_cache"], op.ins["v_cache"], op.ins["pos"]
    Hq, Hkv, d = int(op.attrs["heads"]), int(op.attrs["kv_heads"]), int(op.attrs["head_dim"])
    G, S, C = Hq // Hkv, kc.rows, op.tile["bq"]
    NC, W = _cdiv(S, C), d + 4
    pt = g.tensor(f"attention partials of op {oi}", "f32", (1, NC, Hq, W), "intermediate")
    pos_box = g.full(ps.tensor)
    pos_box = tuple((a, b) for a, b in zip(pos_box.lo, pos_box.hi))
    parts = []
    for c in range(NC):
        r0, r1 = c * C, min(S, c * C + C)
        for kh in range(Hkv):
            reads = [(q.tensor, q.box(0, 1, kh * G * d, (kh + 1) * G * d)),
                     (kn.tensor, kn.box(0, 1, kh * d, (kh + 1) * d)),
                     (vn.tensor, vn.box(0, 1, kh * d, (kh + 1) * d)),
                     (kc.tensor, kc.box(r0, r1, kh * d, (kh + 1) * d)),
                     (vc.tensor, vc.box(r0, r1, kh * d, (kh + 1) * d)),
                     (ps.tensor, pos_box)]
            writes = [(pt, ((0, 1), (c, c + 1), (kh * G, (kh + 1) * G), (0, W)))]
            parts.append(Instr((c, kh, 0, 0), reads, writes))
    o = g.full(op.out)
    comb = []
    for kh in range(Hkv):
        comb.append(Instr((kh, 0, 0, 0),
                          [(pt, ((0, 1), (0, NC), (kh * G, (kh + 1) * G), (0, W))), (ps.tensor, pos_box)],
                          [(op.out, o.box(0, 1, kh * G * d, (kh + 1) * G * d))]))
    return [Node(oi, ATTN_PARTIAL, 0, pt, [q, kn, vn, kc, vc, ps], parts),
            Node(oi, ATTN_COMBINE, 0, op.out, [g.full(pt), ps], comb)]


def _position_column(p: int, hd: int, rope_cols: int) -> int:
    """Output column of packed-tile position p."""
    if hd and p < rope_cols:
        h, w = divmod(p, hd)
        return h * hd + w // 2 + (w % 2) * (hd // 2)
    return p


def _column_runs(p0: int, p1: int, hd: int, rope_cols: int) -> List[Tuple[int, int]]:
    """Columns of positions [p0, p1), merged into maximal [c0, c1) runs."""
    cols = sorted(_position_column(p, hd, rope_cols) for p in range(p0, p1))
    runs: List[List[int]] = []
    for c in cols:
        if runs and runs[-1][1] == c:
            runs[-1][1] = c + 1
        else:
            runs.append([c, c + 1])
    return [(a, b) for a, b in runs]


def _lower_packed_gemv(g: Graph, oi: int, op: Op) -> List[Node]:
    A, B = op.ins["a"], op.ins["b"]
    M, K = A.rows, A.cols
    fl = op.flags
    N = g.tensors[op.out].padded[3]
    t = op.tile
    bm, bn = t["bm"], t["bn"]
    hd = int(op.attrs.get("head_dim", 0)) if fl & ROPE else 0
    rope_cols = int(op.attrs.get("rope_cols", 0) or N) if fl & ROPE else 0
    out = g.full(op.out)
    gamma, bias, res = op.ins.get("gamma"), op.ins.get("bias"), op.ins.get("residual")
    ins = []
    for tm in range(_cdiv(M, bm)):
        for tn in range(_cdiv(N, bn)):
            r0, r1 = tm * bm, min(M, tm * bm + bm)
            runs = _column_runs(tn * bn, min(N, tn * bn + bn), hd, rope_cols)
            reads = [(A.tensor, A.box(r0, r1, 0, K))]
            reads += [(B.tensor, B.box(0, K, c0, c1)) for c0, c1 in runs]
            if fl & SILU_MUL:
                reads += [(B.tensor, B.box(0, K, N + c0, N + c1)) for c0, c1 in runs]
            if fl & RMSNORM_INPUT:
                reads.append((gamma.tensor, gamma.box(0, 1, 0, K)))
            if fl & BIAS:
                reads += [(bias.tensor, bias.box(r0, r1, c0, c1)) for c0, c1 in runs]
            if fl & RESIDUAL:
                reads += [(res.tensor, res.box(r0, r1, c0, c1)) for c0, c1 in runs]
            writes = [(op.out, out.box(r0, r1, c0, c1)) for c0, c1 in runs]
            ins.append(Instr((tm, tn, 0, 0), reads, writes))
    edges = [A, B] + [e for e in (gamma, bias, res) if e is not None]
    return [Node(oi, GEMV, fl, op.out, edges, ins)]


def _grouped_tiles(TM: int, TN: int, S: int, ncu: int) -> List[Tuple[int, int]]:
    """GEMM tile order: the tile grid cut into gm x gn groups, groups taken
    row by row, tiles row by row inside each group."""
    if TM == 0 or TN == 0:
        return []
    B = ncu // 8 if ncu % 8 == 0 else 32
    gm = min(TM, 32)
    gn = min(TN, max(1, B // (gm * S)))
    order = []
    for gi in range(_cdiv(TM, gm)):
        for gj in range(_cdiv(TN, gn)):
            rows = [tm for tm in range(TM) if tm // gm == gi]
            cols = [tn for tn in range(TN) if tn // gn == gj]
            order += [(tm, tn) for tm in rows for tn in cols]
    return order


def _lower_gemm(g: Graph, oi: int, op: Op, ncu: int = 256) -> List[Node]:
    if op.tile.get("gemv", 0) and op.tile.get("layout", 0) == 2:
        return _lower_packed_gemv(g, oi, op)
    A, B = op.ins["a"], op.ins["b"]
    M, K = A.rows, A.cols
    fl = op.flags
    N = g.tensors[op.out].padded[3]
    Nb = 2 * N if fl & SILU_MUL else N
    assert B.rows == K and B.cols == Nb, "B view must be [K, Nb]"
    t = op.tile
    bm, bn, S = t["bm"], t["bn"], t.get("split", 1)
    dup = t.get("dup", 1)
    opcode = GEMV if t.get("gemv", 0) else GEMM
    chunks = _chunks(K, S)
    out = g.full(op.out)
    gamma = op.ins.get("gamma")
    bias = op.ins.get("bias")
    res = op.ins.get("residual")
    if S > 1:
        pt = g.tensor(f"{g.tensors[op.out].name}.partial", "f32", (S, M, Nb),
                      "intermediate")
        P = g.full(pt)
    ins = []
    TM, TN = _cdiv(M, bm), _cdiv(N, bn)
    if opcode == GEMM:
        tiles = _grouped_tiles(TM, TN, S, ncu)
    else:
        tiles = [(tm, tn) for tm in range(TM) for tn in range(TN)]
    for tm, tn in tiles:
        if True:
            r0, r1 = tm * bm, min(M, tm * bm + bm)
            c0, c1 = tn * bn, min(N, tn * bn + bn)
            for s, (k0, k1) in enumerate(chunks):
                reads = [(A.tensor, A.box(r0, r1, k0, k1)),
                         (B.tensor, B.box(k0, k1, c0, c1))]
                if fl & SILU_MUL:
                    reads.append((B.tensor, B.box(k0, k1, N + c0, N + c1)))
                if fl & RMSNORM_INPUT:
                    reads.append((gamma.tensor, gamma.box(0, 1, k0, k1)))
                if S == 1:
                    if fl & BIAS:
                        reads.append((bias.tensor, bias.box(r0, r1, c0, c1)))
                    if fl & RESIDUAL:
                        reads.append((res.tensor, res.box(r0, r1, c0, c1)))
                    writes = [(op.out, out.box(r0, r1, c0, c1))]
                else:
                    pb = lambda cc0, cc1: ((0, 1), (s, s + 1), (r0, r1), (cc0, cc1))
                    writes = [(pt, pb(c0, c1))]
                    if fl & SILU_MUL:
                        writes.append((pt, pb(N + c0, N + c1)))
                for r in range(dup):
                    ins.append(Instr((tm, tn, s, r), list(reads), list(writes)))
    edges = [A, B] + [e for e in (gamma, bias, res) if e is not None]
    if S == 1:
        return [Node(oi, opcode, fl, op.out, edges, ins)]
    part = Node(oi, opcode, PARTIAL | (fl & (SILU_MUL | RMSNORM_INPUT)), pt,
                [A, B] + ([gamma] if gamma is not None else []), ins)
    rbm, rbn = t["rbm"], t["rbn"]
    red = []
    for tm in range(_cdiv(M, rbm)):
        for tn in range(_cdiv(N, rbn)):
            r0, r1 = tm * rbm, min(M, tm * rbm + rbm)
            c0, c1 = tn * rbn, min(N, tn * rbn + rbn)
            reads = [(pt, ((0, 1), (0, S), (r0, r1), (c0, c1)))]
            if fl & SILU_MUL:
                reads.append((pt, ((0, 1), (0, S), (r0, r1), (N + c0, N + c1))))
            if fl & BIAS:
                reads.append((bias.tensor, bias.box(r0, r1, c0, c1)))
            if fl & RESIDUAL:
                reads.append((res.tensor, res.box(r0, r1, c0, c1)))
            if fl & RMSNORM_INPUT:
                reads.append((A.tensor, A.box(r0, r1, 0, K)))
            red.append(Instr((tm, tn, 0, 0), reads, [(op.out, out.box(r0, r1, c0, c1))]))
    redges = [P] + [e for e in (bias, res) if e is not None] + (
        [A] if fl & RMSNORM_INPUT else [])
    return [part, Node(oi, REDUCE, fl, op.out, redges, red)]


def _meta(t: Tensor):
    return (t.dtype, t.padded)


def _intersects(a, b) -> bool:
    return all(max(a[d][0], b[d][0]) < min(a[d][1], b[d][1]) for d in range(4))


@dataclasses.dataclass
class Schedule:
    nodes: List[Node]
    n_instr: int
    ncu: int
    records: List[tuple]          # decoded, one per list entry (pads included)
    targets: List[int]            # barrier targets by barrier id
    n_input_barriers: int
    n_reuse_barriers: int
    slots: Dict[int, int]         # tensor id -> slot
    n_slots: int
    reuse_events: List[Tuple[int, int, int]]   # (node, slot, old tensor)
    deps: Dict[int, Dict[int, frozenset]]      # instr -> {producer node: set}

    @property
    def waves(self) -> int:
        return _cdiv(self.n_instr, self.ncu)

    @property
    def zero_fill(self) -> int:
        return self.waves * self.ncu - self.n_instr


def _level_barriers(nodes, deps, n_instr: int) -> Dict[tuple, dict]:
    """Level-synchronous barriers ("Implementing a Mega Kernel for B300",
    section 7, computing the levels).

    The page gives a task the level 1 + max(level of its parents), level 0
    without parents, and runs the levels one after another with a grid-wide
    barrier between them.  Here a task is an instruction and its parents are
    the producer instructions in its dependency sets.  Reading taken for this
    library's fixed placement (instructions run in list order on their CUs):
    an instruction's level is raised to the previous instruction's level
    where it is lower, so every level is a contiguous run of the list.  The
    barrier between levels L - 1 and L becomes one counter: all real
    instructions of level L - 1 arrive, all of level L wait."""
    owner = {}
    for ni, n in enumerate(nodes):
        for j in range(len(n.instrs)):
            owner[n.start + j] = ni
    level = [0] * n_instr
    for i in range(n_instr):
        lv = level[i - 1] if i > 0 else 0
        for producer_set in deps.get(i, {}).values():
            for a in producer_set:
                lv = max(lv, level[a] + 1)
        level[i] = lv
    by_level: Dict[int, List[int]] = {}
    for i in range(n_instr):
        if i in owner:
            by_level.setdefault(level[i], []).append(i)
    keys: Dict[tuple, dict] = {}
    for lv in sorted(by_level):
        if lv == 0:
            continue
        below, here = by_level[lv - 1], by_level[lv]
        keys[("level", lv)] = dict(first=here[0], kind=0, node=owner[below[0]],
                                   arrive=list(below), wait=list(here))
    return keys


def schedule(g: Graph, ncu: int, cluster_size: int = 1, reuse: int = 0,
             sync: str = "tiles") -> Schedule:
    """Derive the full schedule.  ``reuse``: 0 = no pooling, 1 = pool
    intermediates, 2 = pool intermediates and let graph outputs take pooled
    slots (the dispatcher-owned outputs of MegaKittens Internals, sec. 07).
    ``sync``: "tiles" = one counter per (producer node, dependency set);
    "levels" = one counter per level boundary (see ``_level_barriers``)."""
    nodes = lower(g, ncu)
    # phase 1: count and place
    pos = 0
    for n in nodes:
        if n.opcode == GEMM and ncu % 8 == 0 and len(n.instrs) >= ncu:
            pos = _cdiv(pos, ncu // 8) * (ncu // 8)
        n.start = pos
        pos += _cdiv(len(n.instrs), cluster_size) * cluster_size
        n.end = pos
    n_instr = pos
    gidx = lambda n, j: n.start + j

    producer = {n.out: ni for ni, n in enumerate(nodes)}
    readers: Dict[int, List[int]] = {}
    for ni, n in enumerate(nodes):
        for e in n.edges:
            readers.setdefault(e.tensor, [])
            if ni not in readers[e.tensor]:
                readers[e.tensor].append(ni)

    # phase 2: tensor slots
    slots: Dict[int, int] = {}
    used = set(readers) | set(producer)
    for ti, t in enumerate(g.tensors):
        if ti in used and t.role in ("input", "weight"):
            slots[ti] = len(slots)
    n_slots = len(slots)
    pool: List[Tuple[int, tuple, int, int]] = []   # (slot, meta, end, old tensor)
    reuse_events = []
    last_reader = {t: max(rs) for t, rs in readers.items()}
    for ni, n in enumerate(nodes):
        t = g.tensors[n.out]
        take = None
        if reuse and (t.role == "intermediate" or (reuse == 2 and t.role == "output")):
            ok = [p for p in pool if p[1] == _meta(t) and n.start - p[2] >= ncu]
            if ok:
                take = min(ok, key=lambda p: p[0])
        if take is not None:
            pool.remove(take)
            slots[n.out] = take[0]
            reuse_events.append((ni, take[0], take[3]))
        else:
            slots[n.out] = n_slots
            n_slots += 1
        # release intermediates whose last reader is this node
        for tt in sorted({e.tensor for e in n.edges}):
            if (reuse and tt in producer and last_reader[tt] == ni
                    and g.tensors[tt].role == "intermediate"):
                end = max(nodes[r].end for r in readers[tt])
                pool.append((slots[tt], _meta(g.tensors[tt]), end, tt))

    # phase 3: dependency sets by brute force
    deps: Dict[int, Dict[int, frozenset]] = {}
    wb_cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def write_boxes(pi: int):
        if pi not in wb_cache:
            owners, boxes = [], []
            for j, ins in enumerate(nodes[pi].instrs):
                for (_, b) in ins.writes:
                    owners.append(gidx(nodes[pi], j))
                    boxes.append(b)
            wb_cache[pi] = (np.array(owners, dtype=np.int64),
                            np.array(boxes, dtype=np.int64).reshape(-1, 4, 2))
        return wb_cache[pi]

    for ni, n in enumerate(nodes):
        for j, ins in enumerate(n.instrs):
            i = gidx(n, j)
            d: Dict[int, set] = {}
            for (tt, b) in ins.reads:
                if tt not in producer:
                    continue
                pi = producer[tt]
                own, wb = write_boxes(pi)
                bb = np.array(b, dtype=np.int64)
                hit = np.all(np.maximum(wb[:, :, 0], bb[:, 0]) <
                             np.minimum(wb[:, :, 1], bb[:, 1]), axis=1)
                d.setdefault(pi, set()).update(int(x) for x in own[hit])
            deps[i] = {p: frozenset(s) for p, s in d.items() if s}

    # barriers: input barriers keyed by (producer node, set); reuse barriers
    keys: Dict[tuple, dict] = {}
    for i in sorted(deps):
        for p, s in deps[i].items():
            k = ("in", p, s)
            if k not in keys:
                keys[k] = dict(first=i, kind=0, node=p, arrive=sorted(s), wait=[])
            keys[k]["wait"].append(i)
    if sync == "levels":
        keys = _level_barriers(nodes, deps, n_instr)
    elif sync != "tiles":
        raise ValueError(sync)
    for (ni, slot, old) in reuse_events:
        n = nodes[ni]
        arrive = sorted(gidx(nodes[r], j) for r in readers[old]
                        for j in range(len(nodes[r].instrs)))
        wait = [gidx(n, j) for j in range(len(n.instrs))]
        keys[("reuse", ni)] = dict(first=wait[0], kind=1, node=ni, arrive=arrive,
                                   wait=wait)
    order = sorted(keys.values(), key=lambda b: (b["first"], b["kind"], b["node"]))
    targets = [len(b["arrive"]) for b in order]
    src: Dict[int, List[Tuple[int, int]]] = {}
    dst: Dict[int, List[Tuple[int, int]]] = {}
    for bid, b in enumerate(order):
        for i in b["wait"]:
            src.setdefault(i, []).append((bid, len(b["arrive"])))
        sliced = len(b["arrive"]) <= SLICE_MAX
        for rank, i in enumerate(b["arrive"]):
            dst.setdefault(i, []).append((bid, rank if sliced else -1))
            assert i < b["first"], "dependency must point to a lower index"

    records = []
    for n_i, n in enumerate(nodes):
        for j in range(n.end - n.start):
            i = n.start + j
            if j < len(n.instrs):
                s_ = tuple(sorted(src.get(i, [])))
                d_ = tuple(sorted(dst.get(i, [])))
                if len(s_) > MAX_SRC or len(d_) > MAX_DST:
                    raise ValueError(f"instruction {i} exceeds barrier limits")
                records.append((i, i % ncu, i // ncu, n.opcode, n.flags, n_i,
                                n.instrs[j].coords, s_, d_))
            else:
                records.append((i, i % ncu, i // ncu, NOOP, 0, n_i, (0, 0, 0, 0),
                                (), ()))
    # Instructions between nodes (the alignment gap before a GEMM node that
    # starts on an XCD block boundary) are Noops of no node; the library's
    # record encoding gives them node 0.
    covered = {r[0] for r in records}
    records += [(i, i % ncu, i // ncu, NOOP, 0, 0, (0, 0, 0, 0), (), ())
                for i in range(n_instr) if i not in covered]
    records.sort(key=lambda r: r[0])
    return Schedule(nodes, n_instr, ncu, records, targets,
                    sum(1 for b in order if b["kind"] == 0),
                    sum(1 for b in order if b["kind"] == 1),
                    slots, n_slots, reuse_events, deps)


# --- graph descriptions of the workloads -------------------------------------

def mlp3_graph(L: int, M: int, H: int, tile: Dict[str, int], fused: bool = True,
               dtype: str = "f16", names_w_first: bool = False) -> Graph:
    """x = relu(x @ W[i] + b[i]) for i < L.

    ``fused``: one gemm op per layer carrying BIAS|RELU.  Unfused: the nine
    aten ops of MegaKittens Internals section 02 (mm, add, relu per layer),
    with tile dict keys ``gemm`` and ``ew``.  ``names_w_first`` creates the
    inputs in the traced placeholder order (W, x, b) of that section.
    """
    g = Graph()
    if names_w_first:
        W = g.tensor("W", dtype, (L, H, H), "weight")
        x = g.tensor("x", dtype, (M, H), "input")
        b = g.tensor("b", dtype, (L, M, H), "weight")
    else:
        x = g.tensor("x", dtype, (M, H), "input")
        W = g.tensor("W", dtype, (L, H, H), "weight")
        b = g.tensor("b", dtype, (L, M, H), "weight")
    cur = g.full(x)
    for i in range(L):
        last = i == L - 1
        if fused:
            y = g.tensor(f"y{i}", dtype, (M, H), "output" if last else "intermediate")
            g.ops.append(Op("gemm", dict(a=cur, b=g.select0(W, i), bias=g.select0(b, i)),
                            y, BIAS | RELU, dict(tile)))
            cur = g.full(y)
        else:
            mm = g.tensor(f"mm{i}", dtype, (M, H), "intermediate")
            g.ops.append(Op("gemm", dict(a=cur, b=g.select0(W, i)), mm, 0,
                            dict(tile["gemm"])))
            ad = g.tensor(f"add{i}", dtype, (M, H), "intermediate")
            g.ops.append(Op("add", dict(a=g.full(mm), b=g.select0(b, i)), ad, 0,
                            dict(tile["ew"])))
            r = g.tensor(f"relu{i}", dtype, (M, H), "output" if last else "intermediate")
            g.ops.append(Op("relu", dict(a=g.full(ad)), r, 0, dict(tile["ew"])))
            cur = g.full(r)
    return g


def prefill_graph(d: Dict[str, int], tiles: Sequence[Dict[str, int]]) -> Graph:
    """Y = X @ W1; Z = relu(Y @ W2) (fp16)."""
    g = Graph()
    X = g.tensor("X", "f16", (d["m"], d["k"]), "input")
    W1 = g.tensor("W1", "f16", (d["k"], d["n1"]), "weight")
    W2 = g.tensor("W2", "f16", (d["n1"], d["n2"]), "weight")
    Y = g.tensor("Y", "f16", (d["m"], d["n1"]), "intermediate")
    Z = g.tensor("Z", "f16", (d["m"], d["n2"]), "output")
    g.ops.append(Op("gemm", dict(a=g.full(X), b=g.full(W1)), Y, 0, dict(tiles[0])))
    g.ops.append(Op("gemm", dict(a=g.full(Y), b=g.full(W2)), Z, RELU, dict(tiles[1])))
    return g


def decode_gemm_graph(d: Dict[str, int], tiles: Sequence[Dict[str, int]]) -> Graph:
    """Q = X0 @ Wqkv; A = Q[:, :n_q] @ Wo; U = A @ Wup; D = U @ Wdown (fp16)."""
    g = Graph()
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
    g.ops.append(Op("gemm", dict(a=g.full(X0), b=g.full(Wqkv)), Q, 0, dict(tiles[0])))
    g.ops.append(Op("gemm", dict(a=g.cols(Q, 0, d["n_q"]), b=g.full(Wo)), A, 0,
                    dict(tiles[1])))
    g.ops.append(Op("gemm", dict(a=g.full(A), b=g.full(Wup)), U, 0, dict(tiles[2])))
    g.ops.append(Op("gemm", dict(a=g.full(U), b=g.full(Wdn)), D, 0, dict(tiles[3])))
    return g


def decode_graph(d: Dict[str, int], tiles: Sequence[Dict[str, int]]) -> Graph:
    """Decoder layer at batch 1: four GEMV ops with RMSNorm-input, residual
    and SiLU-mul flags (bf16)."""
    g = Graph()
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
    g.ops.append(Op("gemm", dict(a=g.full(x), b=g.full(Wqkv), gamma=g.full(g1)), qkv,
                    RMSNORM_INPUT, dict(tiles[0])))
    g.ops.append(Op("gemm", dict(a=g.cols(qkv, 0, nq), b=g.full(Wo), residual=g.full(x)),
                    h, RESIDUAL, dict(tiles[1])))
    g.ops.append(Op("gemm", dict(a=g.full(h), b=g.full(Wgu), gamma=g.full(g2)), a,
                    RMSNORM_INPUT | SILU_MUL, dict(tiles[2])))
    g.ops.append(Op("gemm", dict(a=g.full(a), b=g.full(Wd), residual=g.full(h)), out,
                    RESIDUAL, dict(tiles[3])))
    return g


def layer_graph(d: Dict[str, int], tiles: Sequence[Dict[str, int]]) -> Graph:
    """Llama-style decoder layer prefill (bf16): rmsnorm; the QKV projection
    as two GEMMs, over Wq and Wkv (the column blocks [Q] and [K | V] of
    Wqkv, held as two weights), with the rotary epilogue on q and k; causal
    GQA attention; O GEMM + residual; rmsnorm; gate_up GEMM with SiLU-mul;
    down GEMM + residual.  ``tiles`` is in op order (8 entries)."""
    g = Graph()
    S, H = d["seq"], d["hidden"]
    Hq, Hkv, hd, I = d["heads"], d["kv_heads"], d["head_dim"], d["inter"]
    nq, nkv = Hq * hd, Hkv * hd
    x = g.tensor("x", "bf16", (S, H), "input")
    g1 = g.tensor("g1", "bf16", (H,), "weight")
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
    att = dict(heads=Hq, kv_heads=Hkv, head_dim=hd, causal=1)
    g.ops.append(Op("rmsnorm", dict(x=g.full(x), gamma=g.full(g1)), xn, 0, dict(tiles[0])))
    g.ops.append(Op("gemm", dict(a=g.full(xn), b=g.full(Wq)), q, ROPE, dict(tiles[1]), dict(att)))
    g.ops.append(Op("gemm", dict(a=g.full(xn), b=g.full(Wkv)), kv, ROPE, dict(tiles[2]), dict(att)))
    g.ops.append(Op("attention", dict(q=g.full(q), k=g.cols(kv, 0, nkv),
                                      v=g.cols(kv, nkv, 2 * nkv)),
                    o, 0, dict(tiles[3]), dict(att)))
    g.ops.append(Op("gemm", dict(a=g.full(o), b=g.full(Wo), residual=g.full(x)), h1,
                    RESIDUAL, dict(tiles[4])))
    g.ops.append(Op("rmsnorm", dict(x=g.full(h1), gamma=g.full(g2)), hn, 0, dict(tiles[5])))
    g.ops.append(Op("gemm", dict(a=g.full(hn), b=g.full(Wgu)), a, SILU_MUL, dict(tiles[6])))
    g.ops.append(Op("gemm", dict(a=g.full(a), b=g.full(Wd), residual=g.full(h1)), out,
                    RESIDUAL, dict(tiles[7])))
    return g


def decode_kv_graph(d: Dict[str, int], tiles: Sequence[Dict[str, int]]) -> Graph:
    """The decode layer with attention over a KV cache (bf16): RMSNorm-input
    QKV GEMV; decode attention of the new token over the cache (q, k_new,
    v_new the [Q | K | V] column blocks of qkv); O + residual; RMSNorm-input
    gate_up with SiLU-mul; down + residual.  ``tiles`` in op order (5)."""
    g = Graph()
    M, H, nq, nkv, I, hd = d["m"], d["hidden"], d["n_q"], d["n_kv"], d["inter"], d["head_dim"]
    x = g.tensor("x", "bf16", (M, H), "input")
    g1 = g.tensor("g1", "bf16", (H,), "weight")
    Wqkv = g.tensor("Wqkv", "bf16", (H, nq + 2 * nkv), "weight")
    Wo = g.tensor("Wo", "bf16", (nq, H), "weight")
    g2 = g.tensor("g2", "bf16", (H,), "weight")
    Wgu = g.tensor("Wgu", "bf16", (H, 2 * I), "weight")
    Wd = g.tensor("Wd", "bf16", (I, H), "weight")
    kc = g.tensor("k_cache", "bf16", (d["s_max"], nkv), "input")
    vc = g.tensor("v_cache", "bf16", (d["s_max"], nkv), "input")
    pos = g.tensor("pos", "i32", (1,), "input")
    qkv = g.tensor("qkv", "bf16", (M, nq + 2 * nkv), "intermediate")
    o = g.tensor("o", "bf16", (M, nq), "intermediate")
    h = g.tensor("h", "bf16", (M, H), "intermediate")
    a = g.tensor("a", "bf16", (M, I), "intermediate")
    out = g.tensor("out", "bf16", (M, H), "output")
    g.ops.append(Op("gemm", dict(a=g.full(x), b=g.full(Wqkv), gamma=g.full(g1)), qkv,
                    RMSNORM_INPUT, dict(tiles[0])))
    g.ops.append(Op("decode_attention",
                    dict(q=g.cols(qkv, 0, nq), k_new=g.cols(qkv, nq, nq + nkv),
                         v_new=g.cols(qkv, nq + nkv, nq + 2 * nkv), k_cache=g.full(kc),
                         v_cache=g.full(vc), pos=g.full(pos)),
                    o, 0, dict(tiles[1]), dict(heads=nq // hd, kv_heads=nkv // hd, head_dim=hd)))
    g.ops.append(Op("gemm", dict(a=g.full(o), b=g.full(Wo), residual=g.full(x)), h,
                    RESIDUAL, dict(tiles[2])))
    g.ops.append(Op("gemm", dict(a=g.full(h), b=g.full(Wgu), gamma=g.full(g2)), a,
                    RMSNORM_INPUT | SILU_MUL, dict(tiles[3])))
    g.ops.append(Op("gemm", dict(a=g.full(a), b=g.full(Wd), residual=g.full(h)), out,
                    RESIDUAL, dict(tiles[4])))
    return g


def workload_graph(workload: str, d: Dict[str, int],
                   tiles: Sequence[Dict[str, int]]) -> Graph:
    if workload == "mlp3":
        return mlp3_graph(d["layers"], d["m"], d["h"], tiles[0])
    return dict(prefill=prefill_graph, decode_gemm=decode_gemm_graph,
                decode=decode_graph, layer=layer_graph,
                decode_kv=decode_kv_graph)[workload](d, tiles)
