"""Per-instruction timing of one megakernel forward.

``capture`` runs one traced forward (``megakernel_run_traced``): thread 0 of
every workgroup stamps the GPU wall clock when it starts an instruction,
when its counters are satisfied, when the tile body ends and after the
release.  ``summarize`` turns the stamps into per-node wait / body /
release times; ``to_perfetto`` writes a Chrome trace with one track per CU
(the intra-kernel timeline idea of "Beating torch.compile with Megakernels
in CuTe DSL", "Intrakernel Profiling").
"""
from __future__ import annotations

import ctypes
import json
from typing import Dict

import numpy as np

from . import _lib as L

OPCODE_NAMES = ["NOOP", "GEMM", "GEMV", "REDUCE", "RMSNORM", "ATTENTION", "EW_ADD", "EW_RELU",
                "ATTN_PARTIAL", "ATTN_COMBINE"]


def wall_clock_khz() -> int:
    v = ctypes.c_int32()
    L.check(L.load().mk_wall_clock_khz(ctypes.byref(v)))
    return v.value


def capture(runner, with_clock: bool = False):
    """One traced forward; returns int64 [n_instr, 4] stamps (0 for Noops),
    and with ``with_clock`` also the core clock in MHz over the run."""
    import torch
    st = runner.plan.stats()
    n = 4 * st.n_iters * st.num_cus + 4 * st.num_cus
    buf = torch.zeros(n, dtype=torch.int64, device=runner.out.device)
    runner.plan.run_traced(runner.run_bufs, buf)
    runner.plan.check()
    torch.cuda.synchronize()
    h = buf.view(-1, 4).cpu().numpy()
    stamps = h[: st.n_instr]
    if not with_clock:
        return stamps
    return stamps, core_clock_mhz(h[st.n_iters * st.num_cus:], wall_clock_khz())


def core_clock_mhz(clk: np.ndarray, khz: int) -> float:
    """Shader-clock ticks over wall-clock ticks, summed over the workgroups
    that recorded both ends ([num_cus, 4]: wall0, shader0, wall1, shader1),
    times the wall-clock rate."""
    ok = (clk[:, 2] > clk[:, 0]) & (clk[:, 3] > clk[:, 1])
    if not ok.any():
        return float("nan")
    dw = float((clk[ok, 2] - clk[ok, 0]).sum())
    ds = float((clk[ok, 3] - clk[ok, 1]).sum())
    return ds / dw * khz / 1000.0


def summarize(plan, tr: np.ndarray, khz: int = 100000) -> Dict:
    w = plan.instructions()
    us = 1000.0 / khz
    live = tr[:, 0] > 0
    t0 = tr[live, 0].min()
    t_end = tr[live, 3].max()
    nodes = {}
    for i in np.nonzero(live)[0]:
        nd = int(w[i, L.W_NODE])
        e = nodes.setdefault(nd, dict(op=OPCODE_NAMES[int(w[i, L.W_OPCODE])], n=0, wait=0.0,
                                      body=0.0, rel=0.0, first=1e30, last=0.0))
        a, b, c, d = (tr[i] - t0) * us
        e["n"] += 1
        e["wait"] += b - a
        e["body"] += c - b
        e["rel"] += d - c
        e["first"] = min(e["first"], a)
        e["last"] = max(e["last"], d)
    for e in nodes.values():
        for k in ("wait", "body", "rel"):
            e[k] = e[k] / e["n"]
    ncu = plan.stats().num_cus
    busy = np.zeros(ncu)
    for i in np.nonzero(live)[0]:
        busy[i % ncu] += (tr[i, 2] - tr[i, 1]) * us
    span = (t_end - t0) * us
    return dict(span_us=span, nodes=nodes, body_util=float(busy.mean() / span) if span else 0.0)


def node_table(plan, tr: np.ndarray, khz: int = 100000) -> str:
    """Markdown table of one traced forward, a row per lowered node: its
    instruction count, when its first instruction started and its last one
    released (us from the first stamp), and the median / 90th percentile of
    the counter wait, the tile body and the release."""
    w = plan.instructions()
    us = 1000.0 / khz
    live = tr[:, 0] > 0
    t0 = tr[live, 0].min()
    rows = ["| node | op | instrs | first start | last release | wait p50 / p90 | "
            "body p50 / p90 / max | release p50 |",
            "|---|---|---|---|---|---|---|---|"]
    for nd in sorted({int(x) for x in w[live, L.W_NODE]}):
        sel = live & (w[:, L.W_NODE] == nd)
        st = tr[sel]
        wait = (st[:, 1] - st[:, 0]) * us
        body = (st[:, 2] - st[:, 1]) * us
        rel = (st[:, 3] - st[:, 2]) * us
        op = OPCODE_NAMES[int(w[sel, L.W_OPCODE][0])]
        rows.append(
            f"| {nd} | {op} | {int(sel.sum())} | {(st[:, 0].min() - t0) * us:.1f} | "
            f"{(st[:, 3].max() - t0) * us:.1f} | {np.percentile(wait, 50):.2f} / "
            f"{np.percentile(wait, 90):.2f} | {np.percentile(body, 50):.2f} / "
            f"{np.percentile(body, 90):.2f} / {body.max():.2f} | {np.percentile(rel, 50):.2f} |")
    return "\n".join(rows)


def to_perfetto(plan, tr: np.ndarray, path: str, khz: int = 100000) -> None:
    w = plan.instructions()
    us = 1000.0 / khz
    live = tr[:, 0] > 0
    t0 = tr[live, 0].min()
    ncu = plan.stats().num_cus
    ev = []
    for i in np.nonzero(live)[0]:
        a, b, c, d = (float(x) for x in (tr[i] - t0) * us)
        name = f"{OPCODE_NAMES[int(w[i, L.W_OPCODE])]} n{int(w[i, L.W_NODE])} #{i}"
        cu = int(i % ncu)
        ev.append(dict(name="wait", ph="X", ts=a, dur=b - a, pid=0, tid=cu))
        ev.append(dict(name=name, ph="X", ts=b, dur=c - b, pid=0, tid=cu))
        ev.append(dict(name="release", ph="X", ts=c, dur=d - c, pid=0, tid=cu))
    with open(path, "w") as f:
        json.dump(dict(traceEvents=ev), f)
