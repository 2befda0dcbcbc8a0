"""Packed column-tile GEMVs on the host: layout queries, argument checks and
the instruction lists against the brute-force schedule oracle."""
import pytest

import workloads
from oracle import schedule as S
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G
from tiled_gemm_graph_amd.graph import Graph
from tests.test_compiler import _oracle_tiles


def test_decode_weights_are_packed_with_documented_sizes():
    d = workloads.default_dims("decode")
    plan = G.build("decode", d).build()
    tiles = plan.op_tiles()
    assert [(t["gemv"], t["layout"]) for t in tiles] == [(1, 2)] * 4
    H, nqkv, I = d["hidden"], d["n_q"] + 2 * d["n_kv"], d["inter"]
    # [tiles][K][w] elements of 2 bytes; w = bn, or 2 * bn with SILU_MUL
    expect = {"Wqkv": (H, nqkv, tiles[0]["bn"], 1), "Wo": (d["n_q"], H, tiles[1]["bn"], 1),
              "Wgu": (H, I, tiles[2]["bn"], 2), "Wd": (I, H, tiles[3]["bn"], 1)}
    for name, (K, N, bn, f) in expect.items():
        assert plan.weight_layout(name) == (True, -(-N // bn) * K * bn * f * 2), name
    assert plan.weight_layout("x") == (False, 0)
    assert plan.weight_layout("g1") == (False, 0)
    # one packed tile per CU, no REDUCE node: 4 nodes, 4 waves
    st = plan.stats()
    assert st.n_nodes == 4 and st.n_iters == 4
    with pytest.raises(L.MkError) as e:
        plan.pack_weight("x", 16, 16, stream=0)
    assert e.value.status == L.MK_E_INVALID


def test_gemv_pack_option():
    d = workloads.default_dims("decode")
    plan = G.build("decode", d).build(pack=1)
    assert [(t["gemv"], t["layout"]) for t in plan.op_tiles()] == [(1, 1)] * 4
    assert plan.packed_weights() == []
    small = workloads.small_dims("decode")
    assert [t["layout"] for t in G.build("decode", small).build().op_tiles()] == [1] * 4
    assert [t["layout"] for t in G.build("decode", small).build(pack=2).op_tiles()] == [2] * 4
    with pytest.raises(L.MkError):
        G.build("decode", small).build(pack=3)


def test_packed_rejects_views_and_shared_weights():
    g = Graph()
    x = g.tensor("x", "bf16", (1, 64), "input")
    w = g.tensor("w", "bf16", (64, 128), "weight")
    y = g.tensor("y", "bf16", (1, 64), "output")
    g.gemm(x, g.cols(w, 0, 64), y, tile=dict(gemv=1, layout=2))
    with pytest.raises(L.MkError):
        g.build()
    g = Graph()
    x = g.tensor("x", "bf16", (1, 64), "input")
    w = g.tensor("w", "bf16", (64, 64), "weight")
    y = g.tensor("y", "bf16", (1, 64), "intermediate")
    z = g.tensor("z", "bf16", (1, 64), "output")
    g.gemm(x, w, y)
    g.gemm(y, w, z)
    plan = g.build(pack=2)
    assert [t["layout"] for t in plan.op_tiles()] == [1, 1]   # w is read by two ops


def _compare(wl, dims, ncu, **opts):
    g = G.build(wl, dims)
    plan = g.build(num_cus=ncu, **opts)
    chosen = _oracle_tiles(plan.op_tiles())
    og = S.workload_graph(wl, dims, chosen)
    sc = S.schedule(og, ncu=ncu)
    got = plan.decoded()
    assert len(got) == len(sc.records)
    for a, b in zip(got, sc.records):
        assert a == b
    assert list(plan.barriers()) == sc.targets


@pytest.mark.parametrize("ncu", [16, 256])
def test_forced_packed_decode_lists_match_oracle(ncu):
    _compare("decode", workloads.small_dims("decode"), ncu, pack=2)


def rope_graph(M, K, N, hd, rope_cols, tile=None):
    """y = rope(x @ W + bias + res) on the first rope_cols columns, then a
    second GEMV reads y[:, :128] (so its dependencies follow the rotation
    pairs of the packed tiles)."""
    g = Graph()
    x = g.tensor("x", "bf16", (M, K), "input")
    W = g.tensor("W", "bf16", (K, N), "weight")
    b = g.tensor("b", "bf16", (M, N), "input")
    r = g.tensor("r", "bf16", (M, N), "input")
    W2 = g.tensor("W2", "bf16", (128, 64), "weight")
    y = g.tensor("y", "bf16", (M, N), "output")
    z = g.tensor("z", "bf16", (M, 64), "output")
    g.gemm(x, W, y, L.EP_BIAS | L.EP_RESIDUAL | L.EP_ROPE, bias=b, residual=r, head_dim=hd,
           rope_cols=rope_cols, tile=tile)
    g.gemm(g.cols(y, 0, 128), W2, z)
    og = S.Graph()
    ox = og.tensor("x", "bf16", (M, K), "input")
    oW = og.tensor("W", "bf16", (K, N), "weight")
    ob = og.tensor("b", "bf16", (M, N), "input")
    orr = og.tensor("r", "bf16", (M, N), "input")
    oW2 = og.tensor("W2", "bf16", (128, 64), "weight")
    oy = og.tensor("y", "bf16", (M, N), "output")
    oz = og.tensor("z", "bf16", (M, 64), "output")
    return g, og, (ox, oW, ob, orr, oW2, oy, oz)


@pytest.mark.parametrize("ncu", [16, 40])
def test_packed_rope_lists_match_oracle(ncu):
    M, K, N, hd, rc = 2, 256, 384, 64, 256
    g, og, (ox, oW, ob, orr, oW2, oy, oz) = rope_graph(M, K, N, hd, rc)
    plan = g.build(num_cus=ncu, pack=2)
    t0, t1 = _oracle_tiles(plan.op_tiles())
    assert t0["layout"] == 2 and t0["bn"] % hd != 0     # tiles cut across heads
    og.ops.append(S.Op("gemm", dict(a=og.full(ox), b=og.full(oW), bias=og.full(ob),
                                    residual=og.full(orr)), oy,
                       S.BIAS | S.RESIDUAL | S.ROPE, t0, dict(head_dim=hd, rope_cols=rc)))
    og.ops.append(S.Op("gemm", dict(a=og.cols(oy, 0, 128), b=og.full(oW2)), oz, 0, t1))
    sc = S.schedule(og, ncu=ncu)
    got = plan.decoded()
    assert len(got) == len(sc.records)
    for a, b in zip(got, sc.records):
        assert a == b
    assert list(plan.barriers()) == sc.targets


def test_position_columns_pair_rotation_partners():
    # the oracle's position map: neighbours (2i, 2i+1) of a head are the
    # columns i and i + hd/2; positions past rope_cols are themselves
    hd = 8
    cols = [S._position_column(p, hd, 16) for p in range(20)]
    assert cols[:8] == [0, 4, 1, 5, 2, 6, 3, 7]
    assert cols[8:16] == [8, 12, 9, 13, 10, 14, 11, 15]
    assert cols[16:] == [16, 17, 18, 19]
    assert S._column_runs(2, 6, hd, 16) == [(1, 3), (5, 7)]
