"""GPU tests that a stale read, a lost release or acquire, or a placement
bug would fail, through the C ABI.

* One plan runs inputs A, B, A (different seeded activations) and each run
  is checked against its own oracle: a consumer that read an intermediate
  before its producer's release would see the previous run's values.
* ``debug_poison`` fills every plan-owned intermediate with NaN before each
  run, so a read of a value not yet written this run shows up as NaN.
* The work queue (``queue=1``) gives the same bytes as the static placement.

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

ACT = dict(mlp3="x", decode="x", prefill="X", decode_gemm="X0", layer="x", decode_kv="x")
ALL = tuple(workloads.WORKLOADS) + tuple(workloads.EXTRA_WORKLOADS)


def _counters_ok(plan, epochs):
    c = plan.read_counters()
    t = plan.barriers().astype(np.int64)
    assert np.array_equal(c, epochs * t), "counters != epoch * target"


@pytest.mark.parametrize("poison,queue", [(0, 0), (1, 0), (1, 1), (1, 2)])
@pytest.mark.parametrize("wl", ALL)
def test_alternating_inputs_each_run_checked(wl, poison, queue):
    d = workloads.small_dims(wl)
    inp_a = workloads.generate(wl, d)
    inp_b = dict(inp_a)
    act = ACT[wl]
    inp_b[act] = workloads.generate(wl, d, seed=1)[act]
    assert not torch.equal(inp_a[act], inp_b[act])
    say(f"[gpu] A/B/A {wl} dims={d} debug_poison={poison} queue={queue}")
    r = G.Runner(wl, d, inp_a, debug_poison=poison, queue=queue)
    ref_a, ref_b = OG.run(wl, inp_a, d), OG.run(wl, inp_b, d)
    outs = []
    for k, (inp, ref) in enumerate(((inp_a, ref_a), (inp_b, ref_b), (inp_a, ref_a))):
        r.bufs[act].copy_(inp[act])
        r.forward()
        r.plan.check()
        torch.cuda.synchronize()
        got = to_np(r.out)
        assert not np.isnan(got).any(), f"run {k}: NaN in the output (a read of an unwritten value)"
        assert_parity(got, ref, G.DTYPE[wl], f"{wl} run {'ABA'[k]}")
        outs.append(r.out.clone())
    assert torch.equal(outs[0], outs[2])
    _counters_ok(r.plan, 3)


@pytest.mark.parametrize("queue", [1, 2])
@pytest.mark.parametrize("wl", ALL)
def test_work_queue_same_bytes_as_static(wl, queue):
    d = workloads.small_dims(wl)
    inp = workloads.generate(wl, d)
    say(f"[gpu] queue={queue} vs static {wl} dims={d}")
    r = G.Runner(wl, d, inp)
    r.forward()
    r.plan.check()
    ref = r.out.clone()
    qp = r.alt_plan(queue=queue)
    for _ in range(3):
        r.out.zero_()
        r.forward(plan=qp)
        qp.check()
        torch.cuda.synchronize()
        assert torch.equal(r.out, ref), "work-queue run differs from the static placement"
    _counters_ok(qp, 3)


@pytest.mark.parametrize("wl,queue", [("decode", 1), ("layer", 1), ("prefill", 2), ("layer", 2)])
def test_work_queue_full_size(wl, queue):
    d = workloads.default_dims(wl)
    inp = workloads.generate(wl, d)
    say(f"[gpu] queue={queue} full size {wl}")
    r = G.Runner(wl, d, inp, queue=queue)
    for _ in range(2):
        r.forward()
        r.plan.check()
    torch.cuda.synchronize()
    assert_parity(to_np(r.out), OG.run(wl, inp, d), G.DTYPE[wl], f"{wl} full, queue={queue}")
    _counters_ok(r.plan, 2)


def test_full_size_layer_poisoned_intermediates():
    d = workloads.default_dims("layer")
    inp = workloads.generate("layer", d)
    say("[gpu] layer full size, debug_poison=1")
    r = G.Runner("layer", d, inp, debug_poison=1)
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    got = to_np(r.out)
    assert not np.isnan(got).any()
    assert_parity(got, OG.layer(inp, d), "bf16", "layer full poisoned")


def test_small_m_gemm_on_produced_b_takes_the_gemm_body():
    # y = x @ W1 (M = 64), then z = v @ y with v [1, 64]: an M = 1 product
    # whose B is an intermediate.  The GEMV body would stream B before its
    # counters clear, so the compiler gives it the GEMM body.
    g = G.Graph()
    x = g.tensor("x", "f16", (64, 64), "input")
    w1 = g.tensor("w1", "f16", (64, 128), "weight")
    v = g.tensor("v", "f16", (1, 64), "input")
    y = g.tensor("y", "f16", (64, 128), "intermediate")
    z = g.tensor("z", "f16", (1, 128), "output")
    g.gemm(x, w1, y)
    g.gemm(v, y, z)
    plan = g.build()
    assert plan.op_tile(1)["gemv"] == 0
    ops = {int(r[3]) for r in plan.decoded() if r[5] == 1}
    assert ops == {L.I_GEMM}
    gen = torch.Generator().manual_seed(3)
    xs = torch.randn(64, 64, generator=gen).half()
    ws = (torch.randn(64, 128, generator=gen) / 8).half()
    vs = torch.randn(1, 64, generator=gen).half()
    say("[gpu] M = 1 GEMM with an intermediate B")
    bufs = {"x": xs.cuda(), "w1": ws.cuda(), "v": vs.cuda(),
            "z": torch.empty(1, 128, dtype=torch.float16, device="cuda")}
    for name in plan.packed_weights():            # the first GEMM may read w1 packed
        dst = torch.empty(plan.weight_layout(name)[1] // 2, dtype=torch.float16, device="cuda")
        plan.pack_weight(name, bufs[name], dst)
        bufs[name] = dst
    for _ in range(2):
        plan.run(bufs)
        plan.check()
    torch.cuda.synchronize()
    yr = (xs.double() @ ws.double()).half().double()
    ref = (vs.double() @ yr).numpy()
    assert_parity(to_np(bufs["z"]), ref, "f16", "v @ (x @ w1)")


def test_megakittens_mlp_bf16_unfused_pooled():
    # The MLP traced on MegaKittens Internals (section 02): three layers of
    # mm, add, relu in bf16 as nine separate ops, with intermediates pooled
    # in reused buffers (reuse = 1) and elementwise instructions of two
    # 128 x 128 halves (256 x 128).  GEMM tiles are ones the GPU body takes
    # (64 x 64, 256 per GEMM: enough instructions between a buffer's last
    # reader and the next producer of its shape for the pool to reuse it
    # on 256 CUs; the page's 512 x 256 duplicated tile is a host profile
    # only).
    d = dict(layers=3, m=1024, h=1024)
    inp = workloads.generate("mlp3", d, dtype=torch.bfloat16)
    tiles = [dict(gemm=dict(bm=64, bn=64, gemv=0), ew=dict(er=256, ec=128))]
    g = G.build("mlp3", d, tiles, fused=False, dtype="bf16")
    plan = g.build(reuse=1)
    st = plan.stats()
    say(f"[gpu] MegaKittens MLP bf16 unfused reuse=1: {st.n_instr} instrs, {st.n_slots} slots, "
        f"{st.n_reuse_barriers} reuse barriers")
    assert st.n_reuse_barriers > 0
    # GEMM nodes on both sides of the cache-invalidation skip: those whose
    # inputs hold their slots alone skip it, the one reading a pooled slot
    # keeps it
    nodes = plan.nodes()
    own = nodes[nodes[:, 0] == L.I_GEMM, L.N_LINES_OWN]
    assert own.any() and not own.all(), own
    ew = [r for r in plan.decoded() if r[3] in (L.I_EW_ADD, L.I_EW_RELU)]
    assert len(ew) == 6 * (1024 // 256) * (1024 // 128)
    bufs = {k: v.cuda().contiguous() for k, v in inp.items()}
    bufs["y2"] = torch.empty(1024, 1024, dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        plan.run(bufs)
        plan.check()
    torch.cuda.synchronize()
    assert_parity(to_np(bufs["y2"]), OG.mlp3(inp), "bf16", "MegaKittens MLP")
    _counters_ok(plan, 2)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_mfma_probe_counts_every_product(dt):
    # The calibration probe (mk_probe_mfma) must really issue its MFMAs.  A
    # 32 x 32 x 16 product summed over its 1024 outputs is sum_k (sum of A's
    # column k) * (sum of B's row k), and a lane holds the same k values of
    # its A and B fragments, so a wave's total follows from the operands
    # alone; with small integers every partial sum is exact in fp32.
    blocks, iters = 2, 3
    say(f"[gpu] mfma probe {dt} blocks={blocks} iters={iters}")
    g = torch.Generator().manual_seed(7)
    v = torch.randint(-2, 3, (blocks * 512, 16, 8), generator=g).double()
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    ops = v.to(tdt).cuda()
    out = torch.empty(blocks * 512, device="cuda")
    lib = L.load()
    code = L.MK_F16 if dt == "f16" else L.MK_BF16
    L.check(lib.mk_probe_mfma(ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                              blocks, iters, code, None))
    torch.cuda.synchronize()
    got = out.cpu().double().view(blocks * 8, 64).sum(1)
    x = v.view(blocks * 8, 2, 32, 16, 8)          # wave, lane half, lane, fragment, element
    col_a = x[:, :, :, :8, :].sum(2)              # wave, half, A fragment, element
    row_b = x[:, :, :, 8:, :].sum(2)              # wave, half, B fragment, element
    pairs = [(0, 0), (1, 3), (2, 6), (3, 1), (4, 4), (5, 7), (6, 2), (7, 5)]
    want = sum((col_a[:, :, a, :] * row_b[:, :, b, :]).sum((1, 2)) for a, b in pairs) * iters
    assert torch.equal(got, want), (got[:4], want[:4])


def test_gemv_then_packed_gemm_in_one_plan():
    # A GEMV node and an independent packed GEMM node in one plan (the
    # four-wave instance with every body): a CU's GEMM tile comes right
    # after its GEMV instruction, while the GEMV's controller wave may still
    # read its sums from LDS and store them.  The GEMM tile must not touch
    # the LDS arena before its own barrier (no weight prefetch in this
    # instance).  Both outputs against the oracle, two runs.
    g = G.Graph()
    v = g.tensor("v", "bf16", (1, 1024), "input")
    w1 = g.tensor("w1", "bf16", (1024, 2048), "weight")
    g.tensor("y1", "bf16", (1, 2048), "output")
    X = g.tensor("X", "bf16", (256, 1024), "input")
    w2 = g.tensor("w2", "bf16", (1024, 4096), "weight")
    g.tensor("y2", "bf16", (256, 4096), "output")
    g.gemm(v, w1, g.ids["y1"])
    g.gemm(X, w2, g.ids["y2"])
    plan = g.build()
    t0, t1 = plan.op_tile(0), plan.op_tile(1)
    assert t0["gemv"] == 1 and t1["gemv"] == 0 and t1["layout"] == 2
    say(f"[gpu] GEMV then packed GEMM: {plan.stats().n_instr} instructions, tiles {t0['bn']} / "
        f"{t1['bm']}x{t1['bn']}")
    gen = torch.Generator().manual_seed(11)
    mk = lambda *s, std=1.0: (torch.randn(*s, generator=gen) * std).to(torch.bfloat16)
    host = dict(v=mk(1, 1024), w1=mk(1024, 2048, std=1024 ** -0.5), X=mk(256, 1024),
                w2=mk(1024, 4096, std=1024 ** -0.5))
    bufs = {k: t.cuda() for k, t in host.items()}
    for name in plan.packed_weights():
        dst = torch.empty(plan.weight_layout(name)[1] // 2, dtype=torch.bfloat16, device="cuda")
        plan.pack_weight(name, bufs[name], dst)
        bufs[name] = dst
    bufs["y1"] = torch.empty(1, 2048, dtype=torch.bfloat16, device="cuda")
    bufs["y2"] = torch.empty(256, 4096, dtype=torch.bfloat16, device="cuda")
    f = lambda t: t.double().numpy()
    ref1 = f(host["v"]) @ f(host["w1"])
    ref2 = f(host["X"]) @ f(host["w2"])
    for run in range(2):
        bufs["y1"].fill_(float("nan"))
        bufs["y2"].fill_(float("nan"))
        plan.run(bufs)
        plan.check()
        torch.cuda.synchronize()
        assert_parity(to_np(bufs["y1"]), ref1, "bf16", f"GEMV run {run}")
        assert_parity(to_np(bufs["y2"]), ref2, "bf16", f"packed GEMM run {run}")
