"""Host compiler (libmk.so) vs the brute-force schedule oracle, plus ABI
guards.  CPU only: megakernel_build needs no GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import workloads
from oracle import schedule as S
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


def test_library_exports_every_declared_symbol():
    lib = L.load()
    text = open(HEADER).read()
    names = re.findall(r"^\s*(?:mk_status|void|const char|int32_t)\s*\**\s*(\w+)\(", text, re.M)
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.EXPORTS) <= set(names)
    assert lib.mk_abi_version() == 5


def test_mfma_probe_rejects_bad_arguments():
    # argument checks come before any device call, so they run without a GPU
    lib = L.load()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    for args in [(None, p, 1, 1, L.MK_F16), (p, None, 1, 1, L.MK_F16), (p, p, 0, 1, L.MK_F16),
                 (p, p, 65536, 1, L.MK_F16), (p, p, 1, 0, L.MK_F16), (p, p, 1, 1, L.MK_F32)]:
        assert lib.mk_probe_mfma(*args, None) == L.MK_E_INVALID, args


def test_struct_layout_matches_decoder(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stddef.h>
#include <stdio.h>
#include "mk.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(mk_instr), sizeof(mk_node),
    offsetof(mk_instr, opcode)/4, offsetof(mk_instr, n_src)/4, offsetof(mk_instr, coord)/4,
    offsetof(mk_instr, r0)/4, offsetof(mk_instr, split_idx)/4, offsetof(mk_instr, src_id)/4,
    offsetof(mk_instr, src_target)/4, offsetof(mk_instr, dst_id)/4, offsetof(mk_instr, dst_rank)/4,
    sizeof(mk_tile), sizeof(mk_op_attrs));
  printf("%zu %zu %zu\\n", sizeof(mk_build_options), sizeof(mk_plan_stats), sizeof(mk_run_error));
  printf("%zu %zu\\n", offsetof(mk_node, layout)/4, offsetof(mk_node, lines_own)/4);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    l1, l2, l3 = subprocess.check_output([str(exe)]).decode().split("\n")[:3]
    assert [int(x) for x in l3.split()] == [L.N_LAYOUT, L.N_LINES_OWN]
    v = [int(x) for x in l1.split()]
    assert v[:2] == [256, 256]
    assert v[2:11] == [L.W_OPCODE, L.W_NSRC, L.W_COORD, L.W_R0, L.W_SPLIT, L.W_SRC_ID,
                       L.W_SRC_TGT, L.W_DST_ID, L.W_DST_RANK]
    assert L.W_DST_RANK + L.MAX_DST == L.INSTR_WORDS
    assert v[11] == ctypes.sizeof(L.Tile) and v[12] == ctypes.sizeof(L.OpAttrs)
    w = [int(x) for x in l2.split()]
    assert w == [ctypes.sizeof(L.BuildOptions), ctypes.sizeof(L.PlanStats),
                 ctypes.sizeof(L.RunError)]


def _gold():
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "megakittens_mlp_schedule.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = [float(x) if "." in x else int(x) for x in v]
    return vals


def test_megakittens_profile_through_libmk():
    tiles = [dict(gemm=dict(bm=512, bn=256, dup=2, gemv=0), ew=dict(er=256, ec=128))]
    g = G.build("mlp3", dict(layers=3, m=1024, h=1024), tiles, fused=False, w_first=True)
    plan = g.build(num_cus=148, cluster_size=2, reuse=2)
    st = plan.stats()
    gv = _gold()
    assert st.n_instr == gv["instructions"][0]
    assert st.n_iters == gv["whole_waves"][0]
    assert st.n_iters * 148 - st.n_instr == gv["zero_filled_slots"][0]
    assert st.n_slots == gv["tensor_slots"][0]
    assert st.n_input_barriers == gv["input_barriers"][0]
    assert st.n_reuse_barriers == gv["reuse_barriers"][0]
    assert st.n_barriers == gv["barriers"][0]
    assert plan.slots()[g.ids["y2"]] == gv["final_relu_slot"][0]
    # and the whole list equals the oracle's derivation
    og = S.mlp3_graph(3, 1024, 1024, dict(gemm=dict(bm=512, bn=256, dup=2),
                                          ew=dict(er=256, ec=128)),
                      fused=False, names_w_first=True)
    sc = S.schedule(og, ncu=148, cluster_size=2, reuse=2)
    assert plan.decoded() == sc.records
    assert list(plan.barriers()) == sc.targets


def _oracle_tiles(tiles):
    out = []
    for t in tiles:
        d = {k: v for k, v in t.items() if v}
        d.setdefault("split", 1)
        out.append(d)
    return out


def _compare(wl, dims, tiles=None, reuse=0, ncu=256, sync=0):
    g = G.build(wl, dims, tiles)
    plan = g.build(num_cus=ncu, reuse=reuse, sync=sync)
    chosen = _oracle_tiles(plan.op_tiles())
    og = S.workload_graph(wl, dims, chosen if wl != "mlp3" else [chosen[0]])
    sc = S.schedule(og, ncu=ncu, reuse=reuse, sync="levels" if sync else "tiles")
    got = plan.decoded()
    assert len(got) == len(sc.records)
    for a, b in zip(got, sc.records):
        assert a == b, (wl, a, b)
    assert list(plan.barriers()) == sc.targets
    slots = plan.slots()
    for ti, t in enumerate(og.tensors):
        if t.name in g.ids and ti in sc.slots:
            assert slots[g.ids[t.name]] == sc.slots[ti], t.name
    st = plan.stats()
    assert st.n_slots == sc.n_slots
    assert st.n_reuse_barriers == sc.n_reuse_barriers
    return plan, sc


@pytest.mark.parametrize("size", ["small", "full"])
def test_decode_kv_lists_match_oracle(size):
    # the decode layer with split-KV attention: partial and combine nodes,
    # the cache and position reads, the partial tensor's dependency sets
    dims = workloads.small_dims("decode_kv") if size == "small" else workloads.default_dims("decode_kv")
    plan, sc = _compare("decode_kv", dims)
    ops = {int(r[3]) for r in plan.decoded()}
    assert {L.I_ATTN_PARTIAL, L.I_ATTN_COMBINE} <= ops
    for bq in (64, 256):
        _compare("decode_kv", dims, tiles=[None, dict(bq=bq)])


@pytest.mark.parametrize("wl", workloads.WORKLOADS)
def test_full_size_lists_match_oracle(wl):
    dims = workloads.default_dims(wl)
    plan, sc = _compare(wl, dims)
    # every counter's arrivals precede its first waiter (deadlock freedom)
    for i, ds in sc.deps.items():
        for st in ds.values():
            assert max(st) < i


@pytest.mark.parametrize("wl", workloads.WORKLOADS)
def test_level_sync_lists_match_oracle(wl):
    # level-synchronous mode, full and reduced sizes, with and without reuse
    for dims, ncu in ((workloads.default_dims(wl), 256), (workloads.small_dims(wl), 16)):
        plan, _ = _compare(wl, dims, ncu=ncu, sync=1)
        # one counter per level boundary: at most one wait per instruction
        assert max(len(rec[7]) for rec in plan.decoded()) <= 1
    _compare(wl, workloads.small_dims(wl), ncu=16, reuse=1, sync=1)


def test_lists_with_alignment_gaps_match_oracle():
    # A GEMM node of at least num_cus instructions starts on a multiple of
    # num_cus / 8, which can leave Noop instructions between two nodes.
    # Whether a plan has such a gap depends on the tile choices, so several
    # placements are compared and at least one must have one.
    n_gaps = 0
    for wl, ncu in (("layer", 24), ("decode_gemm", 32), ("decode_gemm", 64), ("layer", 40)):
        plan, sc = _compare(wl, workloads.small_dims(wl), ncu=ncu)
        covered = set()
        for n in sc.nodes:
            covered |= set(range(n.start, n.end))
        gaps = [i for i in range(sc.n_instr) if i not in covered]
        for i in gaps:
            assert plan.decoded()[i][3] == 0   # Noop
        n_gaps += len(gaps)
    assert n_gaps > 0


def test_sync_option_checked():
    g = G.build("mlp3", workloads.small_dims("mlp3"))
    with pytest.raises(L.MkError):
        g.build(sync=2)


@pytest.mark.parametrize("wl", workloads.WORKLOADS)
@pytest.mark.parametrize("reuse", [0, 1])
def test_small_lists_match_oracle(wl, reuse):
    _compare(wl, workloads.small_dims(wl), reuse=reuse, ncu=16)


def test_explicit_tiles_and_split_gemm_match_oracle():
    d = dict(m=96, k=512, n_qkv=384, n_q=256, n_o=256, n_up=512, n_down=128)
    tiles = [dict(bm=64, bn=128, split=2, rbm=32, rbn=64, gemv=0),
             dict(bm=64, bn=64, gemv=0),
             dict(bm=128, bn=128, split=4, rbm=64, rbn=128, gemv=0),
             dict(bm=32, bn=1, gemv=1, split=1) if False else dict(bm=64, bn=64, gemv=0)]
    _compare("decode_gemm", d, tiles, ncu=32)


def test_algorithmic_counts():
    for wl in workloads.WORKLOADS:
        dims = workloads.default_dims(wl)
        st = G.build(wl, dims).build().stats()
        from oracle import graphs as OG
        assert abs(st.flops - OG.flops(wl, dims)) / OG.flops(wl, dims) < 1e-9
    # decode: weights 436.2 MB plus a few KB of activations
    st = G.build("decode", workloads.default_dims("decode")).build().stats()
    assert 436.2e6 < st.bytes < 436.5e6


# --- negative tests: build must reject what the pages reject ---------------

def test_rejects_non_topological_and_bad_views():
    g = G.Graph()
    x = g.tensor("x", "f16", (64, 64), "input")
    w = g.tensor("w", "f16", (64, 64), "weight")
    y = g.tensor("y", "f16", (64, 64), "intermediate")
    z = g.tensor("z", "f16", (64, 64), "output")
    with pytest.raises(L.MkError) as e:
        g.gemm(y, w, z)            # y is never written before
    assert e.value.status == L.MK_E_INVALID
    with pytest.raises(L.MkError) as e:
        g.view(x, (0, 0, 0, 0), (1, 1, 65, 64))
    assert e.value.status == L.MK_E_INVALID
    with pytest.raises(L.MkError):
        g.gemm(x, w, x)            # output must not be an input
    g.gemm(x, w, y)
    with pytest.raises(L.MkError):
        g.gemm(x, w, y)            # written twice


def test_rejects_shape_mismatch_and_empty_split():
    g = G.Graph()
    x = g.tensor("x", "f16", (64, 128), "input")
    w = g.tensor("w", "f16", (64, 64), "weight")
    z = g.tensor("z", "f16", (64, 64), "output")
    g.gemm(x, w, z)
    with pytest.raises(L.MkError) as e:
        g.build()
    assert e.value.status == L.MK_E_INVALID
    g = G.Graph()
    x = g.tensor("x", "f16", (64, 256), "input")
    w = g.tensor("w", "f16", (256, 64), "weight")
    z = g.tensor("z", "f16", (64, 64), "output")
    g.gemm(x, w, z, tile=dict(bm=64, bn=64, split=8))
    with pytest.raises(L.MkError) as e:
        g.build()
    assert e.value.status == L.MK_E_INVALID


def test_tensor_limit():
    g = G.Graph()
    for i in range(L.MAX_TENSORS):
        g.tensor(f"t{i}", "f16", (8,), "input")
    with pytest.raises(L.MkError) as e:
        g.tensor("one_too_many", "f16", (8,), "input")
    assert e.value.status == L.MK_E_LIMIT


def test_empty_graph_and_empty_rows():
    g = G.Graph()
    plan = g.build()
    assert plan.stats().n_instr == 0
    g = G.Graph()
    x = g.tensor("x", "f16", (0, 64), "input")
    w = g.tensor("w", "f16", (64, 64), "weight")
    z = g.tensor("z", "f16", (0, 64), "output")
    g.gemm(x, w, z, tile=dict(bm=64, bn=64))
    plan = g.build()
    assert plan.stats().n_instr == 0 and plan.stats().n_barriers == 0


def test_unsupported_profile_builds_but_does_not_run():
    # the 512x256 duplicated tiles of the worked example are host-only
    tiles = [dict(gemm=dict(bm=512, bn=256, dup=2), ew=dict(er=256, ec=128))]
    g = G.build("mlp3", dict(layers=3, m=1024, h=1024), tiles, fused=False, w_first=True)
    plan = g.build(num_cus=148, cluster_size=2, reuse=2)
    with pytest.raises(L.MkError) as e:
        plan.run([], stream=0)
    assert e.value.status == L.MK_E_UNSUPPORTED


@pytest.mark.parametrize("wl,reuse", [("decode", 0), ("layer", 0), ("mlp3", 0), ("layer", 1)])
def test_arrival_ranks_slice_counters(wl, reuse):
    # A counter with target <= SLICE_MAX is one slot per arrival: its
    # arrivals carry ranks 0 .. target-1 in instruction order; a larger
    # counter's arrivals carry -1.
    d = workloads.default_dims(wl) if wl in ("decode", "layer") else workloads.small_dims(wl)
    plan = G.build(wl, d).build(num_cus=256, reuse=reuse)
    targets = list(plan.barriers())
    arrivals = {}
    for rec in plan.decoded():
        for (b, rank) in rec[8]:
            arrivals.setdefault(b, []).append((rec[0], rank))
    assert sorted(arrivals) == list(range(len(targets)))
    whole = 0
    for b, arr in arrivals.items():
        assert len(arr) == targets[b]
        ranks = [r for (_, r) in sorted(arr)]
        if targets[b] <= L.SLICE_MAX:
            assert ranks == list(range(targets[b]))
        else:
            whole += 1
            assert ranks == [-1] * targets[b]
    # the full layer's reuse barriers wait on more arrivals than SLICE_MAX
    assert (whole > 0) == (wl == "layer" and reuse == 1)


def test_causal_attention_work_even_across_cus():
    # Each CU's attention blocks add up to about the same number of keys
    # (instruction j and j + num_cus share a CU; runs alternate direction).
    d = workloads.default_dims("layer")
    plan = G.build("layer", d).build(num_cus=256)
    w = plan.instructions()
    att = np.nonzero(w[:, L.W_OPCODE] == L.I_ATTENTION)[0]
    keys = np.zeros(256)
    for i in att:
        keys[i % 256] += w[i, L.W_R0 + 5]          # k1: keys the block visits
    busy = keys[keys > 0]
    assert busy.max() / busy.min() <= 1.15, (busy.min(), busy.max())


def _produced_b_graph(tile=None):
    g = G.Graph()
    x = g.tensor("x", "f16", (64, 64), "input")
    w1 = g.tensor("w1", "f16", (64, 128), "weight")
    v = g.tensor("v", "f16", (1, 64), "input")
    y = g.tensor("y", "f16", (64, 128), "intermediate")
    z = g.tensor("z", "f16", (1, 128), "output")
    g.gemm(x, w1, y)
    g.gemm(v, y, z, tile=tile)
    return g


def test_small_m_gemm_on_a_produced_b_is_not_a_gemv():
    # The GEMV body streams B before the instruction's counters clear, which
    # is only right for weights and inputs: an M = 1 product whose B is an
    # earlier op's output takes the GEMM body, and forcing the GEMV body on
    # it leaves a plan the GPU refuses (stats.reserved = 1: unsupported).
    plan = _produced_b_graph().build()
    assert plan.op_tile(1)["gemv"] == 0
    assert {r[3] for r in plan.decoded() if r[5] == 1} == {L.I_GEMM}
    assert plan.stats().reserved == 0
    forced = _produced_b_graph(tile=dict(gemv=1)).build()
    assert forced.stats().reserved == 1


def _gemm_chain(n_out, widths, reuse=0):
    # x [1024, 64] -> widths[0] -> widths[1] ... -> n_out, row-major tiles
    g = G.Graph()
    cur = g.tensor("x", "f16", (1024, 64), "input")
    k = 64
    for i, wdt in enumerate(list(widths) + [n_out]):
        w = g.tensor(f"w{i}", "f16", (k, wdt), "weight")
        last = i == len(widths)
        y = g.tensor(f"y{i}", "f16", (1024, wdt), "output" if last else "intermediate")
        g.gemm(cur, w, y, tile=dict(layout=1, bm=64, bn=64))   # row-major 64 x 64 tiles
        cur, k = y, wdt
    return g.build(reuse=reuse)


def test_lines_own_marks_gemm_nodes_that_may_skip_the_invalidation():
    # A row-major GEMM node may skip the cache invalidation of its counter
    # waits when every tensor it reads that the run writes is written in
    # whole 128-byte lines in a slot of its own.
    mlp = G.build("mlp3", workloads.default_dims("mlp3"), None).build()
    assert list(mlp.nodes()[:, L.N_LINES_OWN]) == [1, 1, 1]
    # rows of 1000 fp16 values (2000 bytes) end mid-line: the reader of
    # that tensor keeps the invalidation, the first node (inputs only) not
    odd = _gemm_chain(64, [1000])
    assert list(odd.nodes()[:, L.N_LINES_OWN]) == [1, 0]
    # slot reuse: y3 takes y0's slot (node 2's 256 tiles lie between y0's
    # last reader and y3's writer), so the readers of y0 and y3 keep it
    re = _gemm_chain(64, [1024, 1024, 1024, 1024], reuse=1)
    assert re.stats().n_reuse_barriers > 0
    assert list(re.nodes()[:, L.N_LINES_OWN]) == [1, 0, 1, 1, 0]
    # packed tiles, GEMVs and other bodies never carry the mark
    dec = G.build("decode", workloads.default_dims("decode"), None).build()
    assert not dec.nodes()[:, L.N_LINES_OWN].any()


def test_new_build_options_are_validated():
    g = _produced_b_graph()
    for opt, bad in (("queue", 3), ("debug_poison", 2)):
        with pytest.raises(L.MkError):
            g.build(**{opt: bad})
    with pytest.raises(L.MkError):
        g.build(queue=2, num_cus=100)   # per-XCD queues need a multiple of 8
    # the work queue changes no record: same list, same counters
    a, b = g.build(), g.build(queue=1, debug_poison=1)
    assert np.array_equal(a.instructions(), b.instructions())
    assert np.array_equal(a.barriers(), b.barriers())


def test_noalloc_size_limit_checked_before_any_gpu_call():
    # the full decoder layer needs about 150 MB of intermediates, beyond the
    # allocation-free path's 64 MiB: refused with MK_E_LIMIT, no GPU touched
    plan = G.build("layer", workloads.default_dims("layer")).build()
    assert plan.stats().intermediate_bytes > 64 << 20
    with pytest.raises(L.MkError) as ei:
        plan.run_noalloc([0] * 64, stream=0)
    assert ei.value.status == L.MK_E_LIMIT
    assert "64" in str(ei.value) or "67108864" in str(ei.value)


def test_layer_stack_limits():
    # Prefill decoder layers in sequence (8 lowered nodes each).  Up to 48
    # nodes the persistent kernel keeps every node descriptor in LDS; beyond,
    # a window of 48 consecutive ids per workgroup, which must hold the
    # nodes of three consecutive records of a CU: fine for these layers
    # (every node has at least 256 instructions), refused for the work queue.
    d = workloads.default_dims("layer")
    p15 = G.layer_stack(d, 15).build(num_cus=256)      # 120 nodes, 226 slots
    assert p15.stats().n_nodes == 120 and p15.stats().n_slots == 226
    with pytest.raises(L.MkError) as e:
        p15.run([], stream=0)           # no GPU here: any error but "unsupported"
    assert e.value.status != L.MK_E_UNSUPPORTED
    pq = G.layer_stack(d, 7).build(num_cus=256, queue=1)   # 56 nodes
    with pytest.raises(L.MkError) as e:
        pq.run([], stream=0)
    assert e.value.status == L.MK_E_UNSUPPORTED and "static placement" in str(e.value)
    with pytest.raises(L.MkError) as e:
        G.layer_stack(d, 16).build(num_cus=256)         # 257 graph tensors
    assert e.value.status == L.MK_E_LIMIT


def test_node_window_refuses_records_spanning_48_nodes():
    # 60 tiny nodes (one instruction each, placed on CU i mod C): on 4 CUs
    # three consecutive records of a CU span 9 nodes, fine; on 25 CUs CU 0
    # holds nodes 0, 25 and 50, a span of 51 the window refuses
    g = G.Graph()
    cur = g.tensor("x", "f16", (64, 64), "input")
    w = g.tensor("w", "f16", (64, 64), "weight")
    for i in range(60):
        y = g.tensor(f"y{i}", "f16", (64, 64), "output" if i == 59 else "intermediate")
        g.gemm(cur, w, y, 0, tile=dict(bm=64, bn=64, gemv=0))
        cur = y
    ok = g.build(num_cus=4)
    with pytest.raises(L.MkError) as e:
        ok.run([], stream=0)
    assert e.value.status != L.MK_E_UNSUPPORTED
    bad = g.build(num_cus=25)
    with pytest.raises(L.MkError) as e:
        bad.run([], stream=0)
    assert e.value.status == L.MK_E_UNSUPPORTED and "node window" in str(e.value)
