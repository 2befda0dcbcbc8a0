"""megakernel_run_noalloc (the entry point that allocates nothing) against
megakernel_run on the same plan, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input: the fixed
per-GPU array keeps the first call's contents, so the second call must
clear and upload what it needs.  Each output must equal megakernel_run's
bytes (same records, same kernels) and meet the oracle's bound.
"""
import pytest
import torch

import workloads
from oracle import graphs as OG
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G
from tests.gpu_common import assert_parity, say, to_np

pytestmark = pytest.mark.gpu


def _noalloc_vs_run(wl, d, **opts):
    inp = workloads.generate(wl, d)
    say(f"[gpu] noalloc vs run: {wl} dims={d} opts={opts}")
    r = G.Runner(wl, d, inp, **opts)
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    ref = r.out.clone()
    r.out.zero_()
    r.plan.run_noalloc(r.run_bufs)
    r.plan.check()
    torch.cuda.synchronize()
    assert torch.equal(r.out, ref), f"{wl}: allocation-free run differs from megakernel_run"
    assert_parity(to_np(r.out), OG.run(wl, inp, d), G.DTYPE[wl], f"{wl} noalloc")


def test_noalloc_two_calls_second_smaller():
    # first: the full decode-shaped GEMM chain (about 25 MB of intermediates)
    _noalloc_vs_run("decode_gemm", workloads.default_dims("decode_gemm"))
    # then a smaller graph on the same array
    _noalloc_vs_run("decode", workloads.small_dims("decode"))


def test_noalloc_poisoned_queue_run():
    _noalloc_vs_run("mlp3", workloads.small_dims("mlp3"), debug_poison=1, queue=1)


def test_noalloc_refuses_a_plan_beyond_the_array():
    d = workloads.default_dims("layer")
    plan = G.build("layer", d).build()
    with pytest.raises(L.MkError) as ei:
        plan.run_noalloc([0] * 64, stream=0)
    assert ei.value.status == L.MK_E_LIMIT
