"""Benchmark: each workload graph as one persistent megakernel launch per forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

A step is one forward of a whole graph (every instruction of its plan) on
seeded synthetic inputs already resident in HBM.  The default run measures
all five graphs and prints ONE JSON line headlined by the largest, the
prefill GEMM chain (M = 8192, X@W1 then relu(.@W2), fp16); its "graphs"
block carries, per graph: µs per forward, achieved TFLOP/s or GB/s against
the MI355X roofline, the same graph launched one op at a time, the same
plan on the work queue, parity against the CPU oracle (full outputs) and
the oracle timed on the host.  ``--workload NAME`` prints one line for one
graph, ``--all`` one line per graph.

Each graph first runs forwards for WARM_SECONDS (the clock ramps up after
the idle spells of input generation and the oracle), then W untimed and K
timed forwards give the headline value.  The per-op comparison alternates
blocks of K forwards (megakernel, per-op, ...) and compares medians.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/forward + TFLOP/s (% MFMA peak) or GB/s (% HBM) per graph, 1 MI355X"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
NOMINAL_CLOCK_MHZ = 2400.0   # the clock the nominal peak is quoted at
WARM_SECONDS = 1.0          # forwards run before the timed blocks of each graph
AB_ROUNDS = 3               # per-op blocks (and megakernel blocks) in the interleaved comparison

DESCR = {
    "mlp3": "3-layer MLP x=relu(x@W[i]+b[i]), x 1024x1024, fp16",
    "decode": "decoder layer at batch 1: RMSNorm-fused QKV GEMV N=6144, O + residual N=4096, "
              "RMSNorm-fused gate_up N=28672 with SiLU*mul, down K=14336 + residual; hidden 4096, bf16",
    "prefill": "prefill GEMM chain M=8192: X[8192x8192]@W1[8192x8192], then @W2[8192x28672] "
               "with ReLU, fp16",
    "decode_gemm": "decode-shaped GEMM chain M=256, K=8192: QKV N=10240, attn-out N=8192, "
                   "MLP up N=28672, MLP down K=28672, fp16",
    "layer": "Llama-style decoder layer prefill, seq 2048, hidden 4096, 32/8 heads of 128, causal "
             "attention, RMSNorm, rotary, SiLU*mul MLP inter 14336, bf16",
    "decode_kv": "decoder layer at batch 1 with split-KV attention over a 4096-row KV cache (new token "
                 "at position 4095, rotary and append), hidden 4096, 32/8 heads of 128, inter 14336, bf16",
}
BOUND = dict(mlp3="mfma", decode="hbm", prefill="mfma", decode_gemm="hbm", layer="mfma", decode_kv="hbm")
KERNEL = "mk_persistent"
CSRC = os.path.join(ROOT, "tiled_gemm_graph_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """sha256 over the device sources the persistent kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "mk.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the persistent kernel from the committed
    rocprofv3 counter summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    scaled by what the same counters read for a plain copy of known size.
    None when there is no summary or the kernel sources changed since."""
    path = os.path.join(PROFILES, f"{KERNEL}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("- ") and ": " in ln:
                k, v = ln[2:].split(": ", 1)
                kv[k.strip()] = v.strip().strip("`")
    try:
        if kv["kernel_source_sha256"] != kernel_source_hash():
            return None
        return (float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
                + float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])) * 1024.0
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def warm_up(fn, seconds):
    """Run ``fn`` until ``seconds`` of wall time have passed.  The GPU's
    clock ramps up over tens to hundreds of milliseconds after an idle
    spell (input generation, the CPU oracle), and a timed block that starts
    cold reads several percent slow."""
    import torch
    t0 = time.time()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if time.time() - t0 >= seconds:
                return n


def time_forwards(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per forward


def cpu_baseline(workload, dims, inp, budget_s):
    """The oracle as it stands, timed on the host cores on a bounded sample."""
    import numpy as np
    from oracle import graphs as OG
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    rows_total = dims.get("m", dims.get("seq", 1))
    if workload in ("prefill",):
        rows = list(range(16))
        t0 = time.perf_counter()
        n = 0
        while True:
            OG.run(workload, inp, dims, rows=rows)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = (time.perf_counter() - t0) / n * rows_total / len(rows)
        sample = f"{n} oracle runs of {len(rows)} of {rows_total} rows, scaled to all rows"
    else:
        t0 = time.perf_counter()
        n = 0
        while True:
            OG.run(workload, inp, dims)
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = (time.perf_counter() - t0) / n
        sample = f"{n} full oracle forwards"
    return {"value": dt * 1e6, "unit": "us/forward", "cores": int(cores), "kind": "oracle",
            "sample": sample}


def parity(got, ref):
    """rel-Frobenius and max-abs error (with its index) in fp64."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    i = int(np.argmax(d))
    return {"rel_err": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-12)),
            "max_abs_err": float(d.reshape(-1)[i]),
            "max_abs_at": [int(x) for x in np.unravel_index(i, d.shape)]}


def roofline(workload, st, us, traffic):
    gbs = st.bytes / (us * 1e-6) / 1e9
    tfl = st.flops / (us * 1e-6) / 1e12
    if BOUND[workload] == "hbm":
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": traffic}
    return {"bound": "mfma", "achieved": tfl, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": tfl / PEAK_MFMA_TFLOPS, "traffic": traffic}


def bench_graph(workload, steps, warmup, cpu_budget, do_check=True, sync="tiles", queue_ab=True,
                clock=False):
    """Measure one graph: the megakernel, its per-op version, the same plan
    on the work queue; parity against the oracle on the whole output."""
    import torch

    import workloads
    from tiled_gemm_graph_amd import graphs as G
    from tiled_gemm_graph_amd import trace as TR

    dims = workloads.default_dims(workload)
    log(f"[bench] {workload} dims={dims}: drawing inputs")
    inp = workloads.generate(workload, dims)
    r = G.Runner(workload, dims, inp, device="cuda", sync=1 if sync == "levels" else 0)
    st = r.plan.stats()
    log(f"[bench] {workload} plan: {st.n_instr} instructions, {st.n_iters} waves, "
        f"{st.n_barriers} counters")
    r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    res = {"workload": DESCR[workload], "name": workload, "dims": dims,
           "instructions": int(st.n_instr), "counters": int(st.n_barriers), "sync": sync,
           "alg_flops": st.flops, "alg_bytes": st.bytes,
           "dtype": "bf16" if G.DTYPE[workload] == "bf16" else "f16"}
    if do_check:
        from oracle import graphs as OG
        log(f"[bench] {workload}: oracle on the whole output")
        res.update(parity(r.out.float().cpu().numpy(), OG.run(workload, inp, dims)))
        log(f"[bench] {workload} parity: rel {res['rel_err']:.3e} max-abs {res['max_abs_err']:.3e}")
    warm_up(r.forward, WARM_SECONDS)
    ms = time_forwards(r.forward, steps, warmup)
    r.plan.check()
    # megakernel against the per-op launches of the same plan: blocks of
    # `steps` forwards in alternation (M P M P M P), medians of each, so
    # that neither side gets the clock's ramp or drift to itself
    mk_blocks, op_blocks = [ms], []
    for k in range(AB_ROUNDS):
        op_blocks.append(time_forwards(r.forward_per_op, steps, warmup))
        if k < AB_ROUNDS - 1:
            mk_blocks.append(time_forwards(r.forward, steps, warmup))
    r.plan.check()
    ms_op = statistics.median(op_blocks)
    res["us"] = ms * 1e3
    res["ms_per_step"] = ms
    res["per_op_us"] = ms_op * 1e3
    res["speedup_vs_per_op"] = ms_op / statistics.median(mk_blocks)
    res["ab_blocks_us"] = {"megakernel": [round(x * 1e3, 1) for x in mk_blocks],
                           "per_op": [round(x * 1e3, 1) for x in op_blocks]}
    if queue_ab and sync == "tiles":
        for q, key in ((1, "queue_us"), (2, "xcd_queue_us")):
            qp = r.alt_plan(queue=q)
            r.forward(plan=qp)
            qp.check()
            ms_q = time_forwards(lambda: r.forward(plan=qp), steps, warmup)
            qp.check()
            res[key] = ms_q * 1e3
            del qp
    if clock:
        _, mhz = TR.capture(r, with_clock=True)
        res["core_clock_mhz"] = mhz
    res["gbps"] = st.bytes / (res["us"] * 1e-6) / 1e9
    res["tflops"] = st.flops / (res["us"] * 1e-6) / 1e12
    # the counter summaries are taken on the per-tile-counter plans
    res["roofline"] = roofline(workload, st, res["us"], measured_traffic(workload) if sync == "tiles" else None)
    log(f"[bench] {workload}: {res['us']:.1f} us/forward, per-op {res['per_op_us']:.1f}, "
        f"megakernel/per-op blocks {res['ab_blocks_us']['megakernel']} / {res['ab_blocks_us']['per_op']}"
        + (f", queue {res['queue_us']:.1f}, per-XCD queues {res['xcd_queue_us']:.1f}" if "queue_us" in res else ""))
    if cpu_budget > 0:
        log(f"[bench] {workload}: timing the CPU oracle (~{cpu_budget:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(workload, dims, inp, cpu_budget)
    else:
        res["cpu_baseline"] = None
    del r
    torch.cuda.empty_cache()
    return res


def line_for(head, steps, warmup, graphs=None):
    """The driver's JSON line for graph result ``head``."""
    line = {
        "metric": METRIC,
        "value": head["us"],
        "unit": "us/forward",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded torch CPU generator, normal distributions of the workload spec)",
        "config": {"workload": head["workload"], "name": head["name"], "dims": head["dims"],
                   "instructions": head["instructions"], "counters": head["counters"],
                   "sync": head["sync"], "launches_per_forward": 1},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for k in ("per_op_us", "speedup_vs_per_op", "ab_blocks_us", "queue_us", "xcd_queue_us", "rel_err", "max_abs_err", "max_abs_at",
              "gbps", "tflops", "alg_bytes", "alg_flops", "core_clock_mhz"):
        if k in head:
            line[k] = head[k]
    if "core_clock_mhz" in head:
        line["peak_at_measured_clock_tflops"] = PEAK_MFMA_TFLOPS * head["core_clock_mhz"] / NOMINAL_CLOCK_MHZ
    if graphs is not None:
        line["graphs"] = graphs
    return line


def node_trace(workload, warmup):
    """One traced forward of the megakernel after ``warmup`` untraced ones:
    per-node start, end, wait, body and release times (markdown)."""
    import torch

    import workloads
    from tiled_gemm_graph_amd import graphs as G
    from tiled_gemm_graph_amd import trace as TR

    dims = workloads.default_dims(workload)
    r = G.Runner(workload, dims, workloads.generate(workload, dims), device="cuda")
    for _ in range(max(warmup, 1)):
        r.forward()
    r.plan.check()
    torch.cuda.synchronize()
    stamps, mhz = TR.capture(r, with_clock=True)
    khz = TR.wall_clock_khz()
    s = TR.summarize(r.plan, stamps, khz)
    print(f"{workload} ({DESCR[workload]}): traced forward span {s['span_us']:.1f} us, "
          f"mean tile-body occupancy {s['body_util']:.3f}, core clock {mhz:.0f} MHz\n", flush=True)
    print(TR.node_table(r.plan, stamps, khz), flush=True)


def copy_calibration(mib, steps):
    """A plain device copy of known size: reads and writes ``mib`` MiB per
    launch.  Profiling it with the HBM counters gives the scale that turns
    FETCH_SIZE / WRITE_SIZE into bytes."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = time_forwards(lambda: dst.copy_(src), steps, 2)
    assert torch.equal(dst, src)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "gbps": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def mfma_probe(steps):
    """The MFMA rate this part sustains when only MFMAs run (mk_probe_mfma):
    operands held in registers and changing every instruction, drawn like
    the prefill workload's (A ~ N(0, 1), B ~ N(0, 1/8192)), one workgroup of
    eight waves per CU.  Under the power limit this sits well below the
    nominal peak, and it is the ceiling any GEMM body here can reach."""
    import ctypes
    import torch
    from tiled_gemm_graph_amd import _lib as L
    lib = L.load()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4000
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, tdt, code in (("f16", torch.float16, L.MK_F16), ("bf16", torch.bfloat16, L.MK_BF16)):
        g = torch.Generator(device="cuda").manual_seed(0)
        v = torch.randn(blocks * 512, 16, 8, generator=g, device="cuda")
        v[:, 8:, :] /= math.sqrt(8192.0)
        ops = v.to(tdt).contiguous()
        out = torch.empty(blocks * 512, device="cuda")

        def launch():
            L.check(lib.mk_probe_mfma(ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      blocks, iters, code, stream))
        warm_up(launch, WARM_SECONDS)
        ms = time_forwards(launch, steps, 0)
        assert torch.isfinite(out).all()
        tf = blocks * iters * 2097152 / (ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_of_nominal": round(tf / PEAK_MFMA_TFLOPS, 4),
                     "us_per_launch": round(ms * 1e3, 1),
                     "clock_if_pipes_saturated_mhz": round(NOMINAL_CLOCK_MHZ * tf / PEAK_MFMA_TFLOPS)}
    print(json.dumps({"mfma_probe": res, "blocks": blocks, "iters": iters, "steps": steps,
                      "operands": "A ~ N(0,1), B ~ N(0,1/8192), 8 A and 8 B fragments cycled"}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    choices=["mlp3", "decode", "prefill", "decode_gemm", "layer", "decode_kv"],
                    help="one graph only (default: all five in one line, headlined by prefill)")
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle timing budget of the headline graph (the others get a quarter)")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-queue", action="store_true", help="skip the work-queue A/B")
    ap.add_argument("--sync", choices=["tiles", "levels"], default="tiles",
                    help="per-tile dependency counters (default) or one counter per "
                         "level boundary, for A/B comparison")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only time a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the sustained MFMA rate with random operands")
    ap.add_argument("--node-trace", action="store_true",
                    help="with --workload: print the per-node timeline of one traced forward")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the hash of the kernel sources and exit")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the tile-graph "
              "megakernel is a single-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib, args.steps)
        return
    if args.mfma_probe:
        mfma_probe(args.steps)
        return
    if args.node_trace:
        if not args.workload:
            print("--node-trace needs --workload", file=sys.stderr)
            sys.exit(2)
        node_trace(args.workload, args.warmup)
        return
    kw = dict(do_check=not args.no_check, sync=args.sync, queue_ab=not args.no_queue)
    if args.workload:
        res = bench_graph(args.workload, args.steps, args.warmup, args.cpu_seconds, clock=True, **kw)
        print(json.dumps(line_for(res, args.steps, args.warmup)), flush=True)
        return
    order = ["prefill", "decode", "mlp3", "decode_gemm", "layer", "decode_kv"]
    results = {}
    for wl in order:
        head = wl == "prefill"
        results[wl] = bench_graph(wl, args.steps, args.warmup,
                                  args.cpu_seconds if head else args.cpu_seconds / 4,
                                  clock=head, **kw)
        if args.all:
            print(json.dumps(line_for(results[wl], args.steps, args.warmup)), flush=True)
    if not args.all:
        print(json.dumps(line_for(results["prefill"], args.steps, args.warmup, graphs=results)),
              flush=True)


if __name__ == "__main__":
    main()
