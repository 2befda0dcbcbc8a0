"""GPU: the decoder layer with split-KV attention over a KV cache
(MK_OP_DECODE_ATTENTION), through the C ABI, against the oracle.

Every case prints its name and shapes before touching the GPU.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import graphs as OG
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G
from tests.gpu_common import assert_parity, say, to_np

pytestmark = pytest.mark.gpu

WL = "decode_kv"


def _inputs(d, pos, seed=0):
    inp = workloads.generate(WL, dict(d, pos=pos), seed=seed)
    assert int(inp["pos"][0]) == pos
    return inp


def _check_append(r, inp_before, d, pos, ref_parts):
    """Row pos of each cache holds the new k (rotated) and v; every other
    row is untouched."""
    kc = r.bufs["k_cache"].cpu()
    vc = r.bufs["v_cache"].cpu()
    for name, got, ref_row in (("k", kc, ref_parts["k_row"]), ("v", vc, ref_parts["v_row"])):
        before = inp_before[f"{name}_cache"]
        rows = [j for j in range(d["s_max"]) if j != pos]
        assert torch.equal(got[rows], before[rows]), f"{name} cache rows other than {pos} changed"
        row = got[pos].float().numpy().astype(np.float64)
        want = np.asarray(ref_row, np.float64)
        # bf16 storage: within two units in the last place, at the row's scale
        # (a rotated element can cancel to near zero, but its error follows
        # the magnitude of the un-rotated pair: the GPU rotates the bf16 k)
        scale = max(float(np.sqrt(np.mean(want * want))), 1e-6)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), scale))) - 7)
        bad = np.abs(row - want) > 2 * ulp + 1e-6
        assert not bad.any(), f"{name} row {pos}: {int(bad.sum())} elements off"


@pytest.mark.parametrize("pos", [0, 63, 64, 200, 383])
def test_decode_kv_small_parity_and_append(pos):
    d = workloads.small_dims(WL)
    inp = _inputs(d, pos)
    say(f"[gpu] decode_kv small dims={d} pos={pos}")
    r = G.Runner(WL, dict(d, pos=pos), inp)
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    ref, parts = OG.decode_kv(inp, dict(d, pos=pos), return_cache=True)
    assert_parity(to_np(r.out), ref, "bf16", f"decode_kv pos={pos}")
    _check_append(r, inp, d, pos, parts)


def test_decode_kv_two_steps_on_the_updated_cache():
    d = workloads.small_dims(WL)
    p0 = 130
    inp = _inputs(d, p0)
    say(f"[gpu] decode_kv two steps from pos={p0}")
    r = G.Runner(WL, dict(d, pos=p0), inp)
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    # step two: a new token at p0 + 1 reading the cache the GPU appended to
    x2 = workloads.generate(WL, dict(d, pos=p0), seed=5)["x"]
    r.bufs["x"].copy_(x2)
    r.bufs["pos"].fill_(p0 + 1)
    inp2 = dict(inp, x=x2, pos=torch.tensor([p0 + 1], dtype=torch.int32),
                k_cache=r.bufs["k_cache"].cpu().clone(), v_cache=r.bufs["v_cache"].cpu().clone())
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    ref, parts = OG.decode_kv(inp2, dict(d, pos=p0 + 1), return_cache=True)
    assert_parity(to_np(r.out), ref, "bf16", "decode_kv second step")
    _check_append(r, inp2, d, p0 + 1, parts)


def test_decode_kv_chunk_size_does_not_change_the_result():
    # one chunk of 256 keys, or four of 64: the log-sum-exp merge of the
    # chunks equals the unsplit softmax up to fp32 summation order
    d = dict(workloads.small_dims(WL), s_max=256)
    pos = 255
    inp = _inputs(d, pos)
    outs = {}
    for bq in (256, 128, 64):
        say(f"[gpu] decode_kv s_max=256 pos={pos} chunk={bq}")
        tiles = [None, dict(bq=bq)]
        r = G.Runner(WL, dict(d, pos=pos), {k: v.clone() for k, v in inp.items()}, tiles=tiles)
        n_part = sum(1 for rec in r.plan.decoded() if rec[3] == L.I_ATTN_PARTIAL)
        assert n_part == (256 // bq) * (d["n_kv"] // d["head_dim"])
        r.forward()
        r.plan.check()
        torch.cuda.synchronize()
        outs[bq] = to_np(r.out).astype(np.float64)
    for bq in (128, 64):
        diff = np.abs(outs[bq] - outs[256]).max()
        say(f"  chunk {bq} vs one chunk: max |diff| {diff:.3e}")
        assert diff <= 0.02
    assert_parity(outs[64], OG.decode_kv(inp, dict(d, pos=pos)), "bf16", "decode_kv 4 chunks")


def test_decode_kv_per_op_and_queue_same_bytes():
    d = workloads.small_dims(WL)
    pos = 200
    inp = _inputs(d, pos)
    say(f"[gpu] decode_kv per-op / queue vs megakernel pos={pos}")
    r = G.Runner(WL, dict(d, pos=pos), inp)
    r.forward()
    r.plan.check()
    ref = r.out.clone()
    r.out.zero_()
    r.forward_per_op()
    torch.cuda.synchronize()
    assert torch.equal(r.out, ref)
    qp = r.alt_plan(queue=1)
    r.out.zero_()
    r.forward(plan=qp)
    qp.check()
    torch.cuda.synchronize()
    assert torch.equal(r.out, ref)


def test_decode_kv_full_size():
    d = workloads.default_dims(WL)
    pos = d["pos"]
    inp = _inputs(d, pos)
    say(f"[gpu] decode_kv full dims={d}")
    r = G.Runner(WL, d, inp)
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    ref, parts = OG.decode_kv(inp, d, return_cache=True)
    assert_parity(to_np(r.out), ref, "bf16", "decode_kv full")
    _check_append(r, inp, d, pos, parts)
