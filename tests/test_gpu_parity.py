"""GPU parity: the persistent megakernel vs the CPU oracle, through the C ABI.

Every case prints its name and shapes before touching the GPU.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import graphs as OG
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G
from tests.gpu_common import assert_parity, say, to_np

pytestmark = pytest.mark.gpu


def _run(wl, dims, inp, tiles=None, n=1, per_op=False, **opts):
    say(f"[gpu] {wl} dims={dims} tiles={tiles} opts={opts} per_op={per_op}")
    r = G.Runner(wl, dims, inp, tiles=tiles, **opts)
    for _ in range(n):
        r.forward_per_op() if per_op else r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    return r


def _counters_ok(r, epochs):
    c = r.plan.read_counters()
    t = r.plan.barriers().astype(np.int64)
    assert np.array_equal(c, epochs * t), "counters != epoch * target"


def test_tiny_gemm_identity_is_exact():
    # W = I, b = 0: relu(x @ I + 0) must equal relu(x) bit for bit
    d = dict(layers=1, m=64, h=64)
    inp = workloads.generate("mlp3", d)
    inp["W"] = torch.eye(64, dtype=torch.float16).unsqueeze(0).contiguous()
    inp["b"] = torch.zeros_like(inp["b"])
    r = _run("mlp3", d, inp, tiles=[dict(bm=64, bn=64, gemv=0)])
    assert torch.equal(r.out.cpu(), torch.relu(inp["x"]))
    _counters_ok(r, 1)


@pytest.mark.parametrize("tile,h", [(dict(bm=64, bn=64, gemv=0), 256), (dict(bm=128, bn=128, gemv=0), 256),
                                    (dict(bm=64, bn=128, gemv=0), 256), (dict(bm=128, bn=64, gemv=0), 256),
                                    (dict(bm=64, bn=64, gemv=0), 576), (dict(bm=128, bn=128, gemv=0), 576)])
def test_gemm_tiles_vs_oracle(tile, h):
    # h = 256: fewer K steps than the row-major body's load ring is deep;
    # h = 576: nine K steps, one more than the deepest ring
    d = dict(layers=2, m=200, h=h)
    inp = workloads.generate("mlp3", d)
    r = _run("mlp3", d, inp, tiles=[tile])
    assert_parity(to_np(r.out), OG.mlp3(inp), "f16", f"tile {tile} h={h}")
    _counters_ok(r, 1)


@pytest.mark.parametrize("wl", workloads.WORKLOADS)
def test_small_workload_parity(wl):
    d = workloads.small_dims(wl)
    inp = workloads.generate(wl, d)
    r = _run(wl, d, inp, n=2)
    assert_parity(to_np(r.out), OG.run(wl, inp, d), G.DTYPE[wl], wl)
    _counters_ok(r, 2)
    # deterministic: the same bytes on a third run, and from the per-op path
    first = r.out.clone()
    r.forward(); r.plan.check()
    assert torch.equal(first, r.out)
    r.out.zero_()
    r.forward_per_op(); torch.cuda.synchronize()
    assert torch.equal(first, r.out), "per-op launches differ from the megakernel"


def test_decode_residual_chain_exact():
    # Wo = 0 and Wd = 0: h = x and out = h, exactly
    d = workloads.small_dims("decode")
    inp = workloads.generate("decode", d)
    inp["Wo"].zero_(); inp["Wd"].zero_()
    r = _run("decode", d, inp)
    assert torch.equal(r.out.cpu(), inp["x"])


def test_layer_attention_row0_and_rope_identity():
    # The layer's front half with k|v and the attention output as graph
    # outputs: query row 0 sees only key 0, so every head's output row 0 is
    # exactly its kv head's v row 0 (softmax weight 1.0, bf16 in and out);
    # rotary embedding is the identity at position 0, so k row 0 is the
    # unrotated projection, and at later positions it keeps each rotation
    # pair's norm while changing the values.
    d = workloads.small_dims("layer")
    S, H, Hq, Hkv, hd = d["seq"], d["hidden"], d["heads"], d["kv_heads"], d["head_dim"]
    nq, nkv = Hq * hd, Hkv * hd
    inp = workloads.generate("layer", d)
    g = G.Graph()
    x = g.tensor("x", "bf16", (S, H), "input")
    g1 = g.tensor("g1", "bf16", (H,), "weight")
    W = g.tensor("Wqkv", "bf16", (H, nq + 2 * nkv), "weight")
    xn = g.tensor("xn", "bf16", (S, H), "intermediate")
    q = g.tensor("q", "bf16", (S, nq), "intermediate")
    kv = g.tensor("kv", "bf16", (S, 2 * nkv), "output")
    o = g.tensor("o", "bf16", (S, nq), "output")
    g.rmsnorm(x, g1, xn)
    g.gemm(xn, g.cols(W, 0, nq), q, L.EP_ROPE, head_dim=hd, rope_cols=nq)
    g.gemm(xn, g.cols(W, nq, nq + 2 * nkv), kv, L.EP_ROPE, head_dim=hd, rope_cols=nkv)
    g.attention(q, g.cols(kv, 0, nkv), g.cols(kv, nkv, 2 * nkv), o, Hq, Hkv, hd, True)
    say(f"[gpu] layer front half dims={d}")
    plan = g.build()
    bufs = {k: inp[k].cuda() for k in ("x", "g1", "Wqkv")}
    bufs["kv"] = torch.empty(S, 2 * nkv, dtype=torch.bfloat16, device="cuda")
    bufs["o"] = torch.empty(S, nq, dtype=torch.bfloat16, device="cuda")
    plan.run(bufs)
    plan.check()
    torch.cuda.synchronize()
    kvh, oh = bufs["kv"].cpu(), bufs["o"].cpu()
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        assert torch.equal(oh[0, h * hd:(h + 1) * hd], kvh[0, nkv + kh * hd:nkv + (kh + 1) * hd]), h
    _, parts = OG.layer(inp, d, return_parts=True)
    xn_o = parts["xn"].astype(np.float64)
    k_unrot = xn_o @ inp["Wqkv"][:, nq:nq + nkv].float().numpy().astype(np.float64)
    k_gpu = to_np(kvh[:, :nkv]).astype(np.float64)
    assert_parity(k_gpu[0], k_unrot[0], "bf16", "k row 0 (rotation = identity)")
    assert np.abs(k_gpu[1:] - k_unrot[1:]).max() > 0.05   # rotated further down
    half = hd // 2
    kg = k_gpu.reshape(S, Hkv, hd)
    ku = k_unrot.reshape(S, Hkv, hd)
    ng = kg[..., :half] ** 2 + kg[..., half:] ** 2
    nu = ku[..., :half] ** 2 + ku[..., half:] ** 2
    assert np.abs(ng - nu).max() <= 0.05 * max(1.0, float(nu.max()))
    # and the whole attention output against the oracle's
    assert_parity(to_np(oh), parts["o"].reshape(S, nq), "bf16", "attention output")


@pytest.mark.parametrize("wl", ["mlp3", "decode", "decode_gemm", "prefill"])
def test_full_size_parity(wl):
    # whole outputs against the oracle (prefill: 8192 x 28672)
    d = workloads.default_dims(wl)
    inp = workloads.generate(wl, d)
    r = _run(wl, d, inp)
    got = to_np(r.out)
    del r
    assert_parity(got, OG.run(wl, inp, d), G.DTYPE[wl], f"{wl} full")


def test_full_size_layer():
    d = workloads.default_dims("layer")
    inp = workloads.generate("layer", d)
    r = _run("layer", d, inp)
    assert_parity(to_np(r.out), OG.layer(inp, d), "bf16", "layer full")
    _counters_ok(r, 1)


def test_full_size_layer_buffer_reuse():
    # With buffer reuse the layer's reuse barriers wait on more arrivals than
    # L.SLICE_MAX, so they run as single atomic words beside sliced counters.
    d = workloads.default_dims("layer")
    inp = workloads.generate("layer", d)
    r = _run("layer", d, inp, n=2, reuse=1)
    assert r.plan.barriers().max() > L.SLICE_MAX
    assert_parity(to_np(r.out), OG.layer(inp, d), "bf16", "layer full reuse=1")
    _counters_ok(r, 2)


@pytest.mark.parametrize("wl", workloads.WORKLOADS)
def test_level_sync_parity(wl):
    # Level-synchronous plans (one counter per level boundary) compute the
    # same bytes as the per-tile-counter plans.
    d = workloads.small_dims(wl)
    inp = workloads.generate(wl, d)
    r = _run(wl, d, inp, n=2, sync=1)
    assert_parity(to_np(r.out), OG.run(wl, inp, d), G.DTYPE[wl], f"{wl} levels")
    _counters_ok(r, 2)
    t = _run(wl, d, inp)
    assert torch.equal(t.out, r.out), "level-synchronous plan differs from the per-tile plan"


def test_level_sync_full_layer():
    # full-size layer: level counters of 768 and 1792 arrivals exceed the
    # slice cap and run as single atomic words
    d = workloads.default_dims("layer")
    inp = workloads.generate("layer", d)
    r = _run("layer", d, inp, sync=1)
    assert r.plan.barriers().max() > L.SLICE_MAX
    assert_parity(to_np(r.out), OG.layer(inp, d), "bf16", "layer full levels")
    _counters_ok(r, 1)


@pytest.mark.parametrize("h", [256, 1024])
def test_unfused_mlp_elementwise_bodies(h):
    # The nine-op form of the 3-layer MLP (plain GEMM, then the bias add and
    # the ReLU as standalone elementwise instructions), against the oracle's
    # fused definition: the fp16 roundings between the ops stay well inside
    # the fp16 tolerance.
    d = dict(layers=3, m=200 if h == 256 else 1024, h=h)
    inp = workloads.generate("mlp3", d)
    g = G.build("mlp3", d, fused=False)
    say(f"[gpu] unfused mlp3 dims={d}")
    plan = g.build()
    assert sum(1 for r in plan.decoded() if r[3] in (6, 7)) > 0   # EW_ADD / EW_RELU
    bufs = {k: v.cuda().contiguous() for k, v in inp.items()}
    out = torch.empty(d["m"], h, dtype=torch.float16, device="cuda")
    bufs["y2"] = out
    plan.run(bufs)
    plan.check()
    torch.cuda.synchronize()
    assert_parity(to_np(out), OG.mlp3(inp), "f16", f"unfused mlp3 h={h}")
    _counters_ok_plan(plan, 1)


def _counters_ok_plan(plan, epochs):
    c = plan.read_counters()
    t = plan.barriers().astype(np.int64)
    assert np.array_equal(c, epochs * t), "counters != epoch * target"


def test_empty_rows_graph_runs():
    g = G.Graph()
    x = g.tensor("x", "f16", (0, 64), "input")
    w = g.tensor("w", "f16", (64, 64), "weight")
    z = g.tensor("z", "f16", (0, 64), "output")
    g.gemm(x, w, z, tile=dict(bm=64, bn=64))
    plan = g.build()
    xt = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    wt = torch.randn((64, 64), device="cuda").half()
    zt = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    # zero-size tensors may have no address; pass any valid pointer
    plan.run([wt.data_ptr(), wt.data_ptr(), wt.data_ptr()])
    plan.check()


def test_cooperative_launch_same_bytes():
    d = workloads.small_dims("decode")
    inp = workloads.generate("decode", d)
    r0 = _run("decode", d, inp)
    r1 = _run("decode", d, inp, cooperative=1)
    assert torch.equal(r0.out, r1.out)


@pytest.mark.parametrize("bn,split", [(64, 1), (128, 2), (256, 3), (512, 4)])
def test_gemv_tile_shapes(bn, split):
    # odd / even / single-batch weight streams and their hand-over between
    # consecutive GEMV instructions
    d = dict(m=1, hidden=1024, n_q=1024, n_kv=256, inter=1536)
    inp = workloads.generate("decode", d)
    t = dict(gemv=1, bn=bn, split=split)
    tiles = [t, t, dict(t, bn=max(64, bn // 2)), t]   # gate_up reads 2 * bn columns
    r = _run("decode", d, inp, tiles=tiles)
    assert_parity(to_np(r.out), OG.decode(inp, d), "bf16", f"bn={bn} split={split}")
    first = r.out.clone()
    r.out.zero_()
    r.forward_per_op(); torch.cuda.synchronize()
    assert torch.equal(first, r.out)


def test_tiny_spin_limit_gives_up_and_recovers():
    # Counter waits bounded at 1 us give up long before the producers of the
    # next node finish: the run ends (every workgroup exits) with
    # MK_E_DEADLOCK and a record of the wait that gave up; the plan's
    # counters start over from zero, and a plan with the default bound on the
    # same inputs still matches the oracle.
    d = workloads.default_dims("decode")
    inp = workloads.generate("decode", d)
    say("[gpu] decode full, spin_limit_us=1 (bounded waits give up)")
    r = G.Runner("decode", d, inp, spin_limit_us=1)
    r.forward()
    torch.cuda.synchronize()
    # the aborted run has finished: a new run is refused until the check
    with pytest.raises(L.MkError) as ei:
        r.forward()
    assert ei.value.status == L.MK_E_DEADLOCK
    err = L.RunError()
    st = r.plan._lib.mk_plan_check(r.plan._p, r.plan._stream(None), ctypes.byref(err))
    assert st == L.MK_E_DEADLOCK
    assert err.code == L.MK_E_DEADLOCK
    n_bar = len(r.plan.barriers())
    assert 0 <= err.cu < 256 and 0 <= err.instr < r.plan.stats().n_instr
    assert 0 <= err.barrier < n_bar and err.value < err.need
    assert not np.any(r.plan.read_counters())
    say("[gpu] decode full, default bound after the abort")
    r2 = _run("decode", d, inp)
    assert_parity(to_np(r2.out), OG.run("decode", inp, d), "bf16", "decode after the abort")
    _counters_ok(r2, 1)
