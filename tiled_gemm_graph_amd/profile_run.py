"""Take the rocprofv3 evidence of the bench graphs and write the summaries.

    python -m tiled_gemm_graph_amd.profile_run --out gpurun_out/prof [--workloads decode prefill ...]

For each workload, each step a separate child process (the profiler is
started with the program itself after ``--``, from /tmp):

1. kernel trace: ``rocprofv3 --kernel-trace --stats`` over
   ``bench.py --workload W --steps S --warmup K --cpu-seconds 0 --no-check
   --no-queue``; the persistent launches are 1 parity forward, K warmups,
   S timed forwards and one traced forward, and the summary keeps the S
   timed ones (median, min, max) beside the bench line of the same run;
2. HBM counters: one ``--pmc FETCH_SIZE`` run and one ``--pmc WRITE_SIZE``
   run over the bench command, and the same two over a plain 1 GiB device
   copy (``bench.py --copy-mib 1024``), whose known byte count turns the
   counters into bytes;
3. MFMA activity (MFMA-bound graphs): ``--pmc SQ_VALU_MFMA_BUSY_CYCLES
   GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16``
   in a run of its own;
4. per-node timeline: ``bench.py --workload W --node-trace`` (no profiler).

Raw profiler output stays under ``--out``; the markdown summaries go to
``--profiles`` (``mk_persistent_<workload>_{kernel_trace,hbm_counters,
mfma_counters,node_trace}.md``).  bench.py reads the HBM summary back as
``roofline.traffic`` while the kernel sources hash to the recorded value.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

from . import profile_summary as PS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
KERNEL = "mk_persistent"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = 2500.0


def say(msg):
    print(f"[profile_run {time.strftime('%H:%M:%S')}] {msg}", flush=True)


SUMMARIZE_ONLY = False   # --summarize-only: re-read the logs and raw output of an earlier run


def run(cmd, log_path, limit):
    """Run one step from /tmp under its own kill timer; returns (rc, stdout)."""
    if SUMMARIZE_ONLY:
        with open(log_path) as f:
            return 0, f.read()
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(limit)] + cmd
    say("$ " + " ".join(cmd))
    with open(log_path, "w") as lf:
        p = subprocess.run(full, cwd="/tmp", env=env, stdout=subprocess.PIPE, stderr=lf, text=True)
    with open(log_path, "a") as lf:
        lf.write(p.stdout)
    say(f"  exit {p.returncode}")
    return p.returncode, p.stdout


def bench_constants():
    """WARM_SECONDS and AB_ROUNDS of bench.py (read from its source)."""
    out = {}
    with open(BENCH) as f:
        for ln in f:
            for k in ("WARM_SECONDS", "AB_ROUNDS"):
                if ln.startswith(k + " ="):
                    out[k] = float(ln.split("=", 1)[1].split("#")[0]) if k == "WARM_SECONDS" \
                        else int(ln.split("=", 1)[1].split("#")[0])
    return out


def bench_json(stdout):
    for ln in stdout.splitlines()[::-1]:
        ln = ln.strip()
        if ln.startswith("{") and '"metric"' in ln:
            return json.loads(ln)
    return None


def source_hash():
    out = subprocess.run([sys.executable, BENCH, "--source-hash"], stdout=subprocess.PIPE, text=True, check=True)
    return out.stdout.strip()


def fmt_cmd(cmd, limit):
    """The command as run, with the repository shown at /root/repo (the
    checkout may sit elsewhere with /root/repo linked to it)."""
    txt = " ".join(["timeout", "-s", "KILL", str(limit)] + cmd).replace(ROOT, "/root/repo")
    return "cd /tmp && export TMPDIR=/tmp\n" + txt


def kernel_trace(wl, out, prof, steps, warmup, h):
    d = os.path.join(out, f"kt_{wl}")
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", d, "-o", "run", "--",
           "python3", BENCH, "--workload", wl, "--steps", str(steps), "--warmup", str(warmup),
           "--cpu-seconds", "0", "--no-check", "--no-queue"]
    rc, so = run(cmd, os.path.join(out, f"kt_{wl}.log"), 600)
    line = bench_json(so)
    dur = PS.kernel_durations(d, KERNEL)
    node = PS.kernel_durations(d, "mk_node_kernel")
    if not dur or line is None:
        say(f"  no kernel trace for {wl} (rc {rc})")
        return None
    # persistent launches: parity forward, the warm-up of WARM_SECONDS, then
    # AB_ROUNDS blocks of warmup + steps forwards (the first is the headline
    # block), then one traced forward; keep the timed `steps` of each block
    rounds = bench_constants()["AB_ROUNDS"]
    blk = warmup + steps
    end = len(dur) - 1
    sel = []
    for j in range(rounds):
        stop = end - (rounds - 1 - j) * blk
        sel += [x[1] / 1000.0 for x in dur[stop - steps:stop]]
    med = statistics.median(sel)
    n_nodes = stats_of(wl)["nodes"]
    per_fwd_node = []
    if node and n_nodes and len(node) % n_nodes == 0:
        # every per-op forward launches the plan's non-empty nodes in order
        body = [x[1] / 1000.0 for x in node]
        for k in range(n_nodes):
            per_fwd_node.append(statistics.median(body[k::n_nodes]))
    rf = line.get("roofline", {})
    with open(os.path.join(prof, f"{KERNEL}_{wl}_kernel_trace.md"), "w") as f:
        f.write(f"# {KERNEL} — {wl}: {line['config']['workload']}, kernel trace\n\n")
        f.write("Command (the repository at /root/repo):\n\n```\n" + fmt_cmd(cmd, 600) + "\n```\n\n")
        f.write(f"Persistent launches in launch order: 1 parity forward, the forwards of a one-second warm-up, "
                f"{rounds} blocks of {warmup} untimed and {steps} timed forwards (alternating with blocks of "
                f"per-op forwards), 1 traced forward. The timed launches of the {rounds} blocks:\n\n")
        f.write("| kernel | timed dispatches | median us | min us | max us |\n|---|---|---|---|---|\n")
        f.write(f"| {KERNEL} | {len(sel)} | {med:.1f} | {min(sel):.1f} | {max(sel):.1f} |\n\n")
        f.write(f"Bench line of the same run (HIP events on the launch stream over the timed region, under "
                f"the profiler, which adds a per-dispatch cost that weighs on the per-op launches): "
                f"{line['value']:.1f} us/forward; per-op launches {line.get('per_op_us', float('nan')):.1f} "
                f"us/forward.\n")
        if rf:
            f.write(f"Roofline ({rf['bound']}): {rf['achieved']:.1f} {rf['unit']} of {rf['peak']:.0f} = "
                    f"{100 * rf['frac']:.1f} %, from the kernel's median timed launch: ")
            if rf["bound"] == "hbm":
                a = line["alg_bytes"] / (med * 1e-6) / 1e9
                f.write(f"{a:.1f} GB/s = {100 * a / PEAK_HBM_GBS:.1f} % "
                        f"(algorithmic bytes per forward {line['alg_bytes']:.4e}).\n")
            else:
                a = line["alg_flops"] / (med * 1e-6) / 1e12
                f.write(f"{a:.1f} TFLOP/s = {100 * a / PEAK_MFMA_TFLOPS:.1f} % "
                        f"(algorithmic flops per forward {line['alg_flops']:.4e}).\n")
        if "core_clock_mhz" in line:
            f.write(f"Core clock over the traced forward: {line['core_clock_mhz']:.0f} MHz.\n")
        if per_fwd_node:
            f.write(f"\nPer-op launches (`mk_node_kernel`, {n_nodes} per forward), median duration of each "
                    f"node's launches over the {len(node) // n_nodes} per-op forwards of the run, us: "
                    + ", ".join(f"{x:.1f}" for x in per_fwd_node) + f" (sum {sum(per_fwd_node):.1f}).\n")
        f.write(f"\nKernel source sha256 (`python bench.py --source-hash`): `{h}`\n")
    say(f"  {wl}: persistent median {med:.1f} us, bench {line['value']:.1f} us")
    return dict(median_us=med, clock_mhz=line.get("core_clock_mhz"))


def pmc_pass(tag, counters, prog, out, limit=180):
    d = os.path.join(out, f"pmc_{tag}")
    cmd = ["rocprofv3", "--pmc"] + counters + ["--output-format", "csv", "-d", d, "-o", "run", "--"] + prog
    rc, _ = run(cmd, os.path.join(out, f"pmc_{tag}.log"), limit)
    return rc, d, cmd


def mean_counter(d, name, kernel, big_only=False):
    """Mean of a counter over the dispatches of ``kernel`` (with
    ``big_only``, over those within half of the largest value: the copy
    calibration run also issues a few tiny copies)."""
    c = PS.counters(d, kernel)
    vals = [v[name] for _, v in c.items() if name in v]
    if vals and big_only:
        top = max(vals)
        vals = [v for v in vals if v >= 0.5 * top]
    return (statistics.mean(vals), len(vals), (max(vals) - min(vals)) / max(statistics.mean(vals), 1e-9)) \
        if vals else (None, 0, 0.0)


def copy_scales(out):
    prog = ["python3", BENCH, "--copy-mib", "1024", "--steps", "3"]
    rf, df, cf = pmc_pass("fetch_copy", ["FETCH_SIZE"], prog, out)
    rw, dw, cw = pmc_pass("write_copy", ["WRITE_SIZE"], prog, out)
    fk, _, _ = mean_counter(df, "FETCH_SIZE", "copyBuffer", big_only=True)
    wk, _, _ = mean_counter(dw, "WRITE_SIZE", "copyBuffer", big_only=True)
    if not fk or not wk:
        return None
    return dict(fetch=1048576.0 / fk, write=1048576.0 / wk, fetch_kib=fk, write_kib=wk, cmds=(cf, cw))


def hbm_counters(wl, out, prof, scales, h, alg_bytes):
    prog = ["python3", BENCH, "--workload", wl, "--steps", "3", "--warmup", "1", "--cpu-seconds", "0",
            "--no-check", "--no-queue"]
    rf, df, cf = pmc_pass(f"fetch_{wl}", ["FETCH_SIZE"], prog, out)
    rw, dw, cw = pmc_pass(f"write_{wl}", ["WRITE_SIZE"], prog, out)
    # persistent dispatches: parity, warmup, 3 timed, traced; keep all but the traced one
    fk, nf, sf = mean_counter(df, "FETCH_SIZE", KERNEL)
    wk, nw, sw = mean_counter(dw, "WRITE_SIZE", KERNEL)
    if fk is None or wk is None:
        say(f"  no HBM counters for {wl}")
        return None
    tot = fk * scales["fetch"] + wk * scales["write"]
    mb = tot * 1024 / 1e6
    with open(os.path.join(prof, f"{KERNEL}_{wl}_hbm_counters.md"), "w") as f:
        f.write(f"# {KERNEL} — {wl}: HBM bytes per launch\n\n")
        f.write("Two counter passes over the bench command, each in its own run, and the same two passes "
                "over a plain 1 GiB device copy (`bench.py --copy-mib 1024`, a copy dispatch that reads "
                "and writes exactly 1 GiB) that turns the counters into bytes:\n\n```\n")
        for c in (cf, cw) + scales["cmds"]:
            f.write(fmt_cmd(c, 180) + "\n")
        f.write("```\n\n| dispatch | FETCH_SIZE KiB | WRITE_SIZE KiB |\n|---|---|---|\n")
        f.write(f"| {KERNEL}, {wl} (mean of {nf} / {nw}; spread {100 * sf:.2f} % / {100 * sw:.2f} %) | "
                f"{fk:.2f} | {wk:.2f} |\n")
        f.write(f"| copy 1 GiB | {scales['fetch_kib']:.2f} | {scales['write_kib']:.2f} |\n\n")
        f.write(f"Scale: a 1 GiB copy reads and writes 1048576 KiB, so FETCH_SIZE is scaled by "
                f"{scales['fetch']:.5f} and WRITE_SIZE by {scales['write']:.5f}.\n\n")
        ratio = tot * 1024 / alg_bytes if alg_bytes else float("nan")
        f.write(f"Per persistent launch: {fk:.2f} x {scales['fetch']:.5f} + {wk:.2f} x {scales['write']:.5f} = "
                f"{tot:.0f} KiB = {mb:.1f} MB of HBM traffic, against {alg_bytes / 1e6:.1f} MB of "
                f"algorithmic bytes: {ratio:.3f}x. bench.py reports this figure as `roofline.traffic` while "
                "the kernel sources hash to the value below, and null once they change.\n\n")
        f.write(f"- kernel_source_sha256: {h}\n- fetch_kib_per_dispatch: {fk:.2f}\n"
                f"- fetch_scale: {scales['fetch']:.5f}\n- write_kib_per_dispatch: {wk:.2f}\n"
                f"- write_scale: {scales['write']:.5f}\n")
    say(f"  {wl}: {mb:.1f} MB per launch ({ratio:.2f}x algorithmic)")
    return tot


def mfma_counters(wl, out, prof, h, alg_flops, kt):
    prog = ["python3", BENCH, "--workload", wl, "--steps", "1", "--warmup", "0", "--cpu-seconds", "0",
            "--no-check", "--no-queue"]
    names = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_F16",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    rc, d, cmd = pmc_pass(f"mfma_{wl}", names, prog, out)
    vals = {n: mean_counter(d, n, KERNEL) for n in names}
    if vals["SQ_VALU_MFMA_BUSY_CYCLES"][0] is None:
        say(f"  no MFMA counters for {wl}")
        return
    busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"][0]
    gui = vals["GRBM_GUI_ACTIVE"][0]
    with open(os.path.join(prof, f"{KERNEL}_{wl}_mfma_counters.md"), "w") as f:
        f.write(f"# {KERNEL} — {wl}: MFMA activity\n\nOne counter pass in its own run:\n\n```\n"
                + fmt_cmd(cmd, 180) + "\n```\n\n| counter | mean per persistent dispatch | dispatches |\n|---|---|---|\n")
        for n in names:
            v = vals[n]
            if v[0] is not None:
                f.write(f"| {n} | {v[0]:.4e} | {v[1]} |\n")
        f.write("\n")
        if kt and kt.get("clock_mhz"):
            cyc = kt["median_us"] * kt["clock_mhz"]
            f.write(f"MFMA busy fraction = busy cycles / (1024 SIMDs x the kernel's median timed duration "
                    f"{kt['median_us']:.1f} us x the core clock {kt['clock_mhz']:.0f} MHz of the kernel-trace "
                    f"run) = {100 * busy / (1024.0 * cyc):.1f} % of SIMD cycles.\n")
        if gui:
            # summed over the 8 XCDs; for a short kernel it also counts the profiler's set-up around it
            f.write(f"Against GRBM_GUI_ACTIVE / 8 XCDs instead (the whole counted window): "
                    f"{100 * busy / (gui / 8.0 * 1024.0):.1f} %.\n")
        mops = (vals["SQ_INSTS_VALU_MFMA_MOPS_F16"][0] or 0.0) + (vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"][0] or 0.0)
        if mops:
            f.write(f"(SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16) x 512 = {mops * 512:.4e} MFMA flops per dispatch "
                    f"against {alg_flops:.4e} algorithmic flops per forward (the counters step in units of "
                    "512 flops).\n")
        f.write(f"\nKernel source sha256: `{h}`\n")


def node_trace(wl, out, prof, h):
    cmd = ["python3", BENCH, "--workload", wl, "--node-trace", "--warmup", "3"]
    rc, so = run(cmd, os.path.join(out, f"nt_{wl}.log"), 300)
    if rc != 0:
        return
    body = "\n".join(ln for ln in so.splitlines() if not ln.startswith("/opt/"))
    with open(os.path.join(prof, f"{KERNEL}_{wl}_node_trace.md"), "w") as f:
        f.write(f"# {KERNEL} — {wl}: per-node timeline of one traced forward\n\n")
        f.write("Thread 0 of every workgroup stamps the wall clock (100 MHz) when it takes an instruction, "
                "when its counters clear, when the tile body ends and after the release "
                "(`megakernel_run_traced`). Times in us from the first stamp; 'wait' is start to counters "
                "clear. The stamps add a few stores per instruction to the traced forward.\n\n```\n" + fmt_cmd(cmd, 300) + "\n```\n\n" + body + "\n\n"
                f"Kernel source sha256: `{h}`\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True, help="raw profiler output directory")
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--workloads", nargs="+",
                    default=["prefill", "decode", "mlp3", "decode_gemm", "layer", "decode_kv"])
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--skip", nargs="*", default=[], choices=["trace", "hbm", "mfma", "nodes"])
    ap.add_argument("--summarize-only", action="store_true",
                    help="write the summaries from the logs and raw output already under --out")
    ap.add_argument("--source-hash", default=None,
                    help="with --summarize-only: the kernel-source hash the raw output was taken on")
    a = ap.parse_args(argv)
    global SUMMARIZE_ONLY
    SUMMARIZE_ONLY = a.summarize_only
    out = os.path.abspath(a.out)
    os.makedirs(out, exist_ok=True)
    os.makedirs(a.profiles, exist_ok=True)
    h = a.source_hash if (a.summarize_only and a.source_hash) else source_hash()
    say(f"kernel sources {h[:16]}..., workloads {a.workloads}")
    scales = None if "hbm" in a.skip else copy_scales(out)
    bound = dict(mlp3="mfma", decode="hbm", prefill="mfma", decode_gemm="hbm", layer="mfma", decode_kv="hbm")
    ok = True
    for wl in a.workloads:
        say(f"== {wl}")
        kt = None
        if "trace" not in a.skip:
            kt = kernel_trace(wl, out, a.profiles, a.steps, a.warmup, h)
            ok &= kt is not None
        if "nodes" not in a.skip:
            node_trace(wl, out, a.profiles, h)
        st = stats_of(wl)
        if scales and "hbm" not in a.skip:
            hbm_counters(wl, out, a.profiles, scales, h, st["bytes"])
        if bound[wl] == "mfma" and "mfma" not in a.skip:
            mfma_counters(wl, out, a.profiles, h, st["flops"], kt)
    return 0 if ok else 1


def stats_of(wl):
    """Algorithmic bytes and flops of a workload's plan (host only)."""
    sys.path.insert(0, ROOT)
    import workloads
    from . import _lib as L
    from . import graphs as G
    d = workloads.default_dims(wl)
    plan = G.build(wl, d).build(num_cus=256)
    st = plan.stats()
    w = plan.instructions()
    live = w[:, L.W_OPCODE] != L.I_NOOP
    return dict(bytes=float(st.bytes), flops=float(st.flops), nodes=len(set(w[live, L.W_NODE].tolist())))


if __name__ == "__main__":
    sys.exit(main())
