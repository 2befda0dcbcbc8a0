"""Pins of the instruction-list oracle (CPU only)."""
import os

import numpy as np
import pytest

from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "megakittens_mlp_schedule.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        vals[k] = [float(x) if "." in x else int(x) for x in v]
    return vals


def p3_graph(ew=(256, 128)):
    return S.mlp3_graph(3, 1024, 1024,
                        dict(gemm=dict(bm=512, bn=256, dup=2),
                             ew=dict(er=ew[0], ec=ew[1])),
                        fused=False, dtype="bf16", names_w_first=True)


@pytest.mark.parametrize("ew", [(256, 128), (128, 256)])
def test_megakittens_worked_example(ew):
    gv = _golden()
    sc = S.schedule(p3_graph(ew), ncu=148, cluster_size=2, reuse=2)
    assert sc.n_instr == gv["instructions"][0]
    assert round(sc.n_instr / 148, 2) == gv["waves_fraction"][0]
    assert sc.waves == gv["whole_waves"][0]
    assert sc.zero_fill == gv["zero_filled_slots"][0]
    starts = [n.start for n in sc.nodes]
    ends = [n.end for n in sc.nodes]
    assert ends[1] == gv["layer1_add_end"][0]
    assert starts[7] == gv["layer3_add_start"][0]
    assert starts[8] == gv["final_relu_start"][0]
    assert sc.n_slots == gv["tensor_slots"][0]
    assert sc.slots[sc.nodes[8].out] == gv["final_relu_slot"][0]
    assert sc.n_input_barriers == gv["input_barriers"][0]
    assert sc.n_reuse_barriers == gv["reuse_barriers"][0]
    assert len(sc.targets) == gv["barriers"][0]
    # every barrier a GEMM output feeds (the adds) has target 2 (CTA pairs)
    mm_nodes = {0, 3, 6}
    for i, ds in sc.deps.items():
        for p, st in ds.items():
            if p in mm_nodes:
                assert len(st) == gv["gemm_barrier_target"][0]
    lo, hi = gv["layer2_gemm_rowblock0"]
    relu1 = sc.nodes[2]
    for i in range(lo, hi + 1):
        r = sc.records[i]
        assert r[3] == S.GEMM and r[6][0] == 0
        assert len(sc.deps[i][2]) == gv["layer2_gemm_rowblock0_waits_on"][0]
        # ... exactly the ReLU instructions of rows 0-511
        rows = {relu1.instrs[j - relu1.start].coords[0] for j in sc.deps[i][2]}
        assert rows == {0, 1} if ew[0] == 256 else rows == {0, 1, 2, 3}
    assert sc.records[hi + 1][6][0] == 1


def _last_writer_deps(sc: S.Schedule, g: S.Graph):
    """Per-element last-writer map: the dependency sets of every consumer
    instruction, found element by element (tiny graphs only)."""
    writer = {}
    for ni, n in enumerate(sc.nodes):
        arr = np.full(g.tensors[n.out].padded, -1, dtype=np.int64)
        for j, ins in enumerate(n.instrs):
            for (t, b) in ins.writes:
                sl = tuple(slice(lo, hi) for lo, hi in b)
                arr[sl] = n.start + j
        writer[n.out] = (ni, arr)
    deps = {}
    for ni, n in enumerate(sc.nodes):
        for j, ins in enumerate(n.instrs):
            d = {}
            for (t, b) in ins.reads:
                if t not in writer:
                    continue
                p, arr = writer[t]
                sl = tuple(slice(lo, hi) for lo, hi in b)
                w = set(int(x) for x in np.unique(arr[sl]))
                assert -1 not in w, "read of an element no instruction writes"
                d.setdefault(p, set()).update(w)
            deps[n.start + j] = {p: frozenset(s) for p, s in d.items()}
    return deps


TINY = dict(
    mlp3=(dict(layers=3, m=40, h=48), [dict(bm=16, bn=16)]),
    prefill=(dict(m=40, k=64, n1=48, n2=80),
             [dict(bm=16, bn=16), dict(bm=32, bn=16)]),
    decode_gemm=(dict(m=8, k=128, n_qkv=192, n_q=128, n_o=128, n_up=256, n_down=64),
                 [dict(bm=8, bn=32, split=2, rbm=8, rbn=64), dict(bm=8, bn=64),
                  dict(bm=8, bn=32, split=2, rbm=4, rbn=32), dict(bm=8, bn=16, split=4,
                                                                   rbm=8, rbn=16)]),
    decode=(dict(m=1, hidden=128, n_q=128, n_kv=32, inter=192),
            [dict(bm=1, bn=32, split=2, gemv=1, rbm=1, rbn=64),
             dict(bm=1, bn=64, split=2, gemv=1, rbm=1, rbn=32),
             dict(bm=1, bn=32, split=2, gemv=1, rbm=1, rbn=64),
             dict(bm=1, bn=64, split=3, gemv=1, rbm=1, rbn=64)]),
    layer=(dict(seq=40, hidden=32, heads=4, kv_heads=2, head_dim=8, inter=48),
           [dict(rows=8), dict(bm=16, bn=16), dict(bm=8, bn=16), dict(bq=16),
            dict(bm=16, bn=16), dict(rows=16), dict(bm=16, bn=16), dict(bm=8, bn=16)]),
)


@pytest.mark.parametrize("wl", sorted(TINY))
@pytest.mark.parametrize("reuse", [0, 1])
def test_box_deps_equal_last_writer_map(wl, reuse):
    d, tiles = TINY[wl]
    g = S.workload_graph(wl, d, tiles)
    sc = S.schedule(g, ncu=4, reuse=reuse)
    lw = _last_writer_deps(sc, g)
    for i, ds in sc.deps.items():
        assert ds == lw[i], (wl, i)
    # topological invariant: every counter arrival precedes its first waiter
    for rec in sc.records:
        i, cu, it = rec[0], rec[1], rec[2]
        assert cu == i % 4 and it == i // 4
    for i, ds in sc.deps.items():
        for s in ds.values():
            assert max(s) < i


@pytest.mark.parametrize("wl", sorted(TINY))
def test_level_barriers_order_every_dependency(wl):
    # Level-synchronous mode: following the counters back from an instruction
    # must reach every instruction whose output it reads (the last-writer map,
    # computed without the oracle's dependency sets); every arrival precedes
    # its waiters; each instruction waits on at most one counter.
    d, tiles = TINY[wl]
    g = S.workload_graph(wl, d, tiles)
    sc = S.schedule(g, ncu=4, sync="levels")
    lw = _last_writer_deps(sc, g)
    arrivals = {}
    for rec in sc.records:
        for (b, _) in rec[8]:
            arrivals.setdefault(b, []).append(rec[0])
    before = {}
    for rec in sorted(sc.records):
        i, reached = rec[0], set()
        assert len(rec[7]) <= 1
        for (b, tgt) in rec[7]:
            assert tgt == len(arrivals[b])
            for a in arrivals[b]:
                assert a < i
                reached.add(a)
                reached |= before[a]
        before[i] = reached
    for i, ds in lw.items():
        for st in ds.values():
            assert set(st) <= before[i], (wl, i)


def test_level_barriers_of_a_chain():
    # A 3-layer chain of 4 x 4 tiles: levels 0, 1, 2, so two counters, each
    # with one arrival per tile of the layer below (the page's level rule:
    # one more than the highest parent level).
    g = S.mlp3_graph(3, 64, 64, dict(bm=16, bn=16))
    sc = S.schedule(g, ncu=8, sync="levels")
    assert sc.targets == [16, 16]
    tiles = S.schedule(g, ncu=8)
    assert len(tiles.targets) > 2   # per-tile mode: one counter per row block


def test_reuse_barrier_waits_for_all_old_readers():
    g = S.mlp3_graph(5, 64, 64, dict(bm=16, bn=16))
    sc = S.schedule(g, ncu=8, reuse=1)
    assert sc.n_reuse_barriers >= 1
    for (ni, slot, old) in sc.reuse_events:
        readers = [n for n in sc.nodes if any(e.tensor == old for e in n.edges)]
        assert sc.nodes[ni].start - max(r.end for r in readers) >= 8
        tgt = sum(len(r.instrs) for r in readers)
        first = sc.nodes[ni].start
        assert tgt in [t for (b, t) in sc.records[first][7]]


def test_negative_limits():
    with pytest.raises(ValueError):
        S._chunks(256, 8)           # chunks of 64 -> only 4 non-empty
    assert S._chunks(4096, 3) == [(0, 1408), (1408, 2816), (2816, 4096)]
