"""GPU: packed column-tile GEMVs (layout, parity, rotary epilogue)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import graphs as OG
from oracle import ops
from tiled_gemm_graph_amd import _lib as L
from tiled_gemm_graph_amd import graphs as G
from tests.gpu_common import TOL, max_abs, rel_fro, say, to_np
from tests.test_packed import rope_graph

pytestmark = pytest.mark.gpu


def _expected_packed(W, N, bn, silu, hd, rope_cols):
    """The documented packed layout, built position by position in numpy."""
    K = W.shape[0]
    T = -(-N // bn)
    w = 2 * bn if silu else bn
    out = np.zeros((T, K, w), dtype=W.dtype)
    for t in range(T):
        for j in range(w):
            p = t * bn + (j - bn if silu and j >= bn else j)
            if p >= N:
                continue
            if hd and p < rope_cols:
                h, r = divmod(p, hd)
                col = h * hd + r // 2 + (r % 2) * (hd // 2)
            else:
                col = p
            if silu and j >= bn:
                col += N
            out[t, :, j] = W[:, col]
    return out


def test_pack_kernel_matches_layout():
    d = dict(m=1, hidden=512, n_q=512, n_kv=128, inter=776)   # ragged last gate_up tile
    inp = workloads.generate("decode", d)
    say(f"[gpu] pack layout decode dims={d}")
    g = G.build("decode", d)
    plan = g.build(pack=2)
    for name in ("Wqkv", "Wgu", "Wd"):
        oi = {"Wqkv": 0, "Wo": 1, "Wgu": 2, "Wd": 3}[name]
        t = plan.op_tile(oi)
        src = inp[name].cuda()
        packed, nbytes = plan.weight_layout(name)
        assert packed
        dst = torch.full((nbytes // 2,), 7, dtype=src.dtype, device="cuda")
        plan.pack_weight(name, src, dst)
        torch.cuda.synchronize()
        N = {"Wqkv": d["n_q"] + 2 * d["n_kv"], "Wgu": d["inter"], "Wd": d["hidden"]}[name]
        ref = _expected_packed(inp[name].view(torch.int16).numpy(), N, t["bn"], name == "Wgu", 0, 0)
        got = dst.view(torch.int16).cpu().numpy().reshape(ref.shape)
        assert np.array_equal(got, ref), name


@pytest.mark.parametrize("dims", [workloads.small_dims("decode"),
                                  dict(m=1, hidden=512, n_q=512, n_kv=128, inter=776),
                                  dict(m=3, hidden=512, n_q=512, n_kv=128, inter=768)])
def test_forced_packed_decode_parity(dims):
    inp = workloads.generate("decode", dims)
    say(f"[gpu] packed decode dims={dims}")
    r = G.Runner("decode", dims, inp, pack=2)
    assert [t["layout"] for t in r.plan.op_tiles()] == [2, 2, 2, 2]
    r.forward(); r.forward(); r.plan.check(); torch.cuda.synchronize()
    ref = OG.decode(inp, dims)
    got = to_np(r.out)
    rel = rel_fro(got, ref)
    say(f"  rel={rel:.3e} maxabs={max_abs(got, ref)}")
    assert rel <= TOL["bf16"]
    c = r.plan.read_counters()
    assert np.array_equal(c, 2 * r.plan.barriers().astype(np.int64))
    first = r.out.clone()
    r.out.zero_()
    r.forward_per_op(); torch.cuda.synchronize()
    assert torch.equal(first, r.out)


def test_full_decode_packed_matches_row_major_path():
    d = workloads.default_dims("decode")
    inp = workloads.generate("decode", d)
    say(f"[gpu] full decode packed vs row-major split-K dims={d}")
    rp = G.Runner("decode", d, inp)
    assert [t["layout"] for t in rp.plan.op_tiles()] == [2, 2, 2, 2]
    rr = G.Runner("decode", d, inp, pack=1)
    rp.forward(); rp.plan.check()
    rr.forward(); rr.plan.check()
    torch.cuda.synchronize()
    ref = OG.decode(inp, d)
    for r in (rp, rr):
        rel = rel_fro(to_np(r.out), ref)
        say(f"  rel={rel:.3e}")
        assert rel <= TOL["bf16"]


def _rope_reference(x, W, b, res, hd, rope_cols):
    y = ops.gemm(x, W, dt=np.float64) + b.astype(np.float64) + res.astype(np.float64)
    M = y.shape[0]
    lead = y[:, :rope_cols].reshape(M, rope_cols // hd, hd)
    # positions of the rows are 0 .. M-1
    rot = ops.rope(lead, dt=np.float64).reshape(M, rope_cols)
    return np.concatenate([rot, y[:, rope_cols:]], axis=1)


@pytest.mark.parametrize("mode", ["packed", "split", "gemm"])
def test_rope_bias_residual_epilogue(mode):
    M = 64 if mode == "gemm" else 3
    K, N, hd, rc = 256, 384, 64, 256
    tile = {"packed": dict(gemv=1, layout=2), "split": dict(gemv=1, bn=128, split=2, rbn=128),
            "gemm": dict(gemv=0, bm=64, bn=128)}[mode]
    say(f"[gpu] rope+bias+residual mode={mode} M={M} K={K} N={N} hd={hd} rope_cols={rc}")
    g, _, _ = rope_graph(M, K, N, hd, rc, tile=tile)
    plan = g.build()
    gen = torch.Generator().manual_seed(5)
    mk = lambda *s, std=1.0: (torch.randn(*s, generator=gen) * std).to(torch.bfloat16)
    x, W, b, res = mk(M, K), mk(K, N, std=K ** -0.5), mk(M, N), mk(M, N)
    W2 = mk(128, 64, std=128 ** -0.5)
    dev = {n: t.cuda() for n, t in dict(x=x, W=W, b=b, r=res, W2=W2).items()}
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(M, 64, dtype=torch.bfloat16, device="cuda")
    bufs = dict(dev, y=y, z=z)
    for name in plan.packed_weights():
        dst = torch.empty(plan.weight_layout(name)[1] // 2, dtype=torch.bfloat16, device="cuda")
        plan.pack_weight(name, dev[name], dst)
        bufs[name] = dst
    plan.run(bufs)
    plan.check()
    torch.cuda.synchronize()
    f = lambda t: t.float().numpy()
    ref = _rope_reference(f(x), f(W), f(b), f(res), hd, rc)
    got = to_np(y)
    rel = rel_fro(got, ref)
    say(f"  y rel={rel:.3e} maxabs={max_abs(got, ref)}")
    assert rel <= TOL["bf16"]
    zref = ops.gemm(got[:, :128], f(W2), dt=np.float64)
    assert rel_fro(to_np(z), zref) <= TOL["bf16"]


def test_full_decode_repeated_runs_identical():
    # packed tiles publish their outputs with write-through stores and no L2
    # write-back: repeated runs must give the same bytes every time
    d = workloads.default_dims("decode")
    inp = workloads.generate("decode", d)
    say(f"[gpu] full decode x40 dims={d}")
    r = G.Runner("decode", d, inp)
    r.forward(); r.plan.check(); torch.cuda.synchronize()
    first = r.out.clone()
    outs = []
    for _ in range(40):
        r.forward()
        outs.append(r.out.clone())
    r.plan.check(); torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, first)
    c = r.plan.read_counters()
    assert np.array_equal(c, 41 * r.plan.barriers().astype(np.int64))
