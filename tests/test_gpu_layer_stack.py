"""GPU: several prefill decoder layers in one persistent launch (the layer
graph repeated, each layer with its own weights), through the C ABI.

Rounding differences between the GPU (bf16 intermediates) and the oracle
(fp64 inside a layer) grow with depth through random-weight layers, so the
stack is not held to one layer's tolerance against the oracle's own chain.
Instead:

* a one-layer plan is run layer after layer, each on the previous GPU
  output, and every layer's output is compared with the oracle's layer
  applied to that same input (one layer's tolerance);
* the n-layer plan, one launch, must give exactly the bytes of that chain
  (every node has the same shapes and so the same tiles);
* the n-layer plan's per-op launches must give the same bytes again.

Stacks of 8 and 14 layers have more lowered nodes (64, 112) than the
persistent kernel keeps in LDS at once, so they run through its
node-descriptor window.  Every case prints its name and shapes before
touching the GPU.
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


def _bind(plan, n: int, d, per, first: int, x: torch.Tensor, out: torch.Tensor):
    """Device buffers for a plan of n layers whose layer j takes the weights
    of layer first + j."""
    nq = d["heads"] * d["head_dim"]
    bufs = {"x": x}
    for j in range(n):
        inp = per[first + j]
        for k in ("g1", "Wo", "g2", "Wgu", "Wd"):
            bufs[f"{k}_{j}"] = inp[k].cuda().contiguous()
        bufs[f"Wq_{j}"] = inp["Wqkv"][:, :nq].contiguous().cuda()
        bufs[f"Wkv_{j}"] = inp["Wqkv"][:, nq:].contiguous().cuda()
    for name in plan.packed_weights():
        dst = torch.empty(plan.weight_layout(name)[1] // 2, dtype=torch.bfloat16, device="cuda")
        plan.pack_weight(name, bufs[name], dst)
        bufs[name] = dst
    bufs[f"out_{n - 1}"] = out
    return bufs


@pytest.mark.parametrize("n", [2, 3, 8, 14])
def test_layer_stack_small(n):
    d = workloads.small_dims("layer")
    x, per = _layer_inputs(d, n)
    S, H = d["seq"], d["hidden"]
    one = G.layer_stack(d, 1).build()
    plan = G.layer_stack(d, n).build()
    say(f"[gpu] {n} decoder layers dims={d}: {plan.stats().n_nodes} nodes, "
        f"{plan.stats().n_instr} instructions")

    # the chain of one-layer launches, each layer against the oracle
    cur = x.cuda()
    for l in range(n):
        y = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
        one.run(_bind(one, 1, d, per, l, cur, y))
        one.check()
        torch.cuda.synchronize()
        ref = np.asarray(OG.layer(dict(per[l], x=cur.cpu()), d), np.float32)
        assert_parity(to_np(y), ref, "bf16", f"layer {l} of {n}")
        cur = y

    # the stack in one launch (twice: counters carried over between runs)
    out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    bufs = _bind(plan, n, d, per, 0, x.cuda(), out)
    for _ in range(2):
        plan.run(bufs)
        plan.check()
    torch.cuda.synchronize()
    assert torch.equal(out, cur), (f"{n}-layer launch differs from the one-layer chain: "
                                   f"max |diff| {(out.float() - cur.float()).abs().max().item()}")
    out.zero_()
    plan.run_per_op(bufs)
    torch.cuda.synchronize()
    assert torch.equal(out, cur), "per-op launches differ from the megakernel"
