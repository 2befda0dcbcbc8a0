"""GPU: several prefill decoder layers in one persistent launch (the layer
graph repeated, each layer with its own weights), through the C ABI, against
the oracle's layers applied in sequence.

Each layer's output is stored in bf16 and is the next layer's input, on the
GPU and in the oracle chain alike.  Every case prints its name and shapes
before touching the GPU.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import graphs as OG
from tiled_gemm_graph_amd import graphs as G
from tests.gpu_common import assert_parity, say, to_np

pytestmark = pytest.mark.gpu


def _layer_inputs(d, n):
    """Per layer: that layer's weights drawn with seed l (the layer
    workload's draw); x from seed 0."""
    per = [workloads.generate("layer", d, seed=l) for l in range(n)]
    return per[0]["x"], per


def _oracle_chain(x, per, d):
    cur = x
    for inp in per:
        cur = torch.from_numpy(np.asarray(OG.layer(dict(inp, x=cur), d), np.float32)).to(torch.bfloat16)
    return cur.float().numpy()


@pytest.mark.parametrize("n", [2, 3])
def test_layer_stack_small(n):
    d = workloads.small_dims("layer")
    x, per = _layer_inputs(d, n)
    g = G.layer_stack(d, n)
    plan = g.build()
    say(f"[gpu] {n} decoder layers dims={d}: {plan.stats().n_instr} instructions")
    nq = d["heads"] * d["head_dim"]
    bufs = {"x": x.cuda()}
    for l, inp in enumerate(per):
        for k in ("g1", "Wo", "g2", "Wgu", "Wd"):
            bufs[f"{k}_{l}"] = inp[k].cuda().contiguous()
        bufs[f"Wq_{l}"] = inp["Wqkv"][:, :nq].contiguous().cuda()
        bufs[f"Wkv_{l}"] = inp["Wqkv"][:, nq:].contiguous().cuda()
    for name in plan.packed_weights():
        dst = torch.empty(plan.weight_layout(name)[1] // 2, dtype=torch.bfloat16, device="cuda")
        plan.pack_weight(name, bufs[name], dst)
        bufs[name] = dst
    out = torch.empty(d["seq"], d["hidden"], dtype=torch.bfloat16, device="cuda")
    bufs[f"out_{n - 1}"] = out
    for _ in range(2):
        plan.run(bufs)
        plan.check()
    torch.cuda.synchronize()
    ref = _oracle_chain(x, per, d)
    assert_parity(to_np(out), ref, "bf16", f"{n} layers")
    first = out.clone()
    out.zero_()
    plan.run_per_op(bufs)
    torch.cuda.synchronize()
    assert torch.equal(out, first), "per-op launches differ from the megakernel"
