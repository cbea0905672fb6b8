#!/usr/bin/env python
"""Profiles behind the bench figures, collected with rocprofv3 on one MI355X.

    python profile_bench.py trace   [--out DIR]  # kernel trace + stats of a short bench run   (GPU)
    python profile_bench.py traffic [--out DIR]  # HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (GPU)
    python profile_bench.py mfma    [--out DIR]  # MFMA flops executed and MFMA busy share per launch (GPU)
    python profile_bench.py render  [--out DIR]  # summaries under profiles/ from the raw output (no GPU)
    python profile_bench.py copy                 # (the calibration program the traffic mode profiles)

The GPU modes keep rocprofv3's raw output and their results under the
output directory (``--out DIR``, default ``profile_out/``, not committed);
`render` turns those into the short summaries that are kept under profiles/.

`trace` runs ``rocprofv3 --kernel-trace --stats`` over ``bench.py`` and writes
profiles/prefill64k_decode_kernel_trace.md: the command, the per-kernel
launch statistics and the bench JSON line of the same run.

`traffic` runs one ``rocprofv3 --pmc`` pass per counter (FETCH_SIZE, then
WRITE_SIZE; KiB per dispatch) over a short bench run and over a plain device
copy of a known number of bytes.  The copy's reading calibrates each counter
(factor = bytes moved / bytes counted); the kernels' readings are scaled by
it.  Results go to profiles/traffic.json, keyed by a digest of the kernel
sources (bench.py reports a traffic figure only while the sources are
unchanged), with a readable summary in profiles/traffic_prefill64k_decode.md.

`mfma` runs one ``rocprofv3 --pmc MfmaUtil MfmaFlops MfmaFlopsBF16`` pass over
the same short bench run and writes profiles/mfma_prefill64k.md: per
whole-workload launch of the MFMA kernels, the matrix flops the hardware
executed (the bf16 splits of fp32 operands included), their rate over the
dispatch's duration, the MFMA units' busy share of the whole chip, and for the
state chain the ratio of executed to algorithmic flops.

This script starts rocprofv3 as a child process and touches the GPU only
through it (and through `copy`, which the profiler runs).
"""
from __future__ import annotations

import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(ROOT, "profile_out")  # raw profiler output; set by --out
PROFILES = os.path.join(ROOT, "profiles")
# more specific names first: a kernel is keyed by the first entry its name contains
KERNELS = ("bwd_chain_kernel", "bwd_local_kernel", "bwd_grad_kernel", "bwd_table_kernel", "conv_silu_kernel",
           "conv_decode_kernel", "chain_kr_kernel", "chain_kernel", "intra_kernel", "output_kernel", "decode_kernel", "chunk_table_kernel")
COPY_BYTES = 1 << 30
BENCH_TRACE = ["bench.py", "--steps", "5", "--warmup", "2", "--decode-steps", "32", "--no-cpu-baseline", "--no-other"]
BENCH_PMC = ["bench.py", "--steps", "1", "--warmup", "1", "--decode-steps", "4", "--no-cpu-baseline", "--no-other",
             "--no-backward"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def run_profiler(args, tag, timeout):
    d = os.path.join(OUT, tag)
    os.makedirs(d, exist_ok=True)
    cmd = ["rocprofv3", *args, "-d", d, "-o", "run", "--output-format", "csv", "--", sys.executable]
    log(f"[profile] {tag}: {' '.join(cmd[:-1])} python3 ...")
    env = dict(os.environ, TMPDIR="/tmp")
    return cmd, d, env, timeout


def launch(cmd_tail, prof_args, tag, timeout):
    cmd, d, env, timeout = run_profiler(prof_args, tag, timeout)
    full = cmd + cmd_tail
    with open(os.path.join(d, "stdout.txt"), "w") as so, open(os.path.join(d, "stderr.txt"), "w") as se:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + full, cwd=ROOT, env=env, stdout=so, stderr=se)
    log(f"[profile] {tag}: exit {r.returncode}")
    return r.returncode, d, " ".join(["rocprofv3", *prof_args, "-d", os.path.relpath(d, ROOT), "-o", "run",
                                      "--output-format", "csv", "--", "python3", *cmd_tail])


def kernel_key(name):
    for k in KERNELS:
        if k in name:
            return k
    return None


def find(d, suffix):
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    return hits[0] if hits else None


def finished(d):
    """The profiled program printed its last line (the bench JSON line or 'copied ...')."""
    try:
        with open(os.path.join(d, "stdout.txt")) as f:
            lines = [l for l in f.read().splitlines() if l.strip()]
    except OSError:
        return False
    return bool(lines) and (lines[-1].startswith("{") or lines[-1].startswith("copied"))


def profiler_ok(rc, d, result_suffix):
    """The profiled program exited 0, printed its last line, and the result
    file exists.  Any other exit, the profiler's own included, is a failure."""
    return rc == 0 and find(d, result_suffix) is not None and finished(d)


def mode_trace():
    rc, d, cmd = launch(BENCH_TRACE, ["--kernel-trace", "--stats"], "trace", 900)
    with open(os.path.join(d, "command.txt"), "w") as f:
        f.write(cmd + "\n")
    if not profiler_ok(rc, d, "kernel_stats.csv"):
        raise SystemExit(f"trace run failed (exit {rc})")


def render_trace():
    d = os.path.join(OUT, "trace")
    stats = find(d, "kernel_stats.csv")
    if stats is None:
        log("[profile] no trace output to render")
        return
    cmd = open(os.path.join(d, "command.txt")).read().strip()
    bench_line = ""
    with open(os.path.join(d, "stdout.txt")) as f:
        for line in f:
            if line.startswith("{"):
                bench_line = line.strip()
    rows = []
    with open(stats) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
                         float(r["Percentage"])))
    lines = ["# Kernel trace: 64K-token prefill (H=6, d=256, bf16), batched decode, front end, prefill backward", "",
             "Command (repository root, one MI355X):", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | {pct:.1f} |")
    lines += ["", "Bench JSON line of the same run:", "", "```", bench_line, "```", ""]
    path = os.path.join(PROFILES, "prefill64k_decode_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[profile] wrote {path}")


def full_launch(name, grid, groups):
    """True for the dispatch group that covers the whole workload: the
    chain instance launched once over all chunks on its own (the stage-by-stage
    run, as timed for the roofline); for the decode kernel the d_v = 256 batch
    (the smaller of its two grids: the bench also times a d_v = 512 batch);
    else the largest grid of the kernel."""
    if kernel_key(name).startswith("bwd_"):
        return True  # the backward has no segmented launches
    if kernel_key(name) == "chain_kr_kernel":
        return ", false, false>" in name  # neither a window/segment launch nor the pipelined one
    if kernel_key(name) == "chain_kernel":
        return ", false>" in name
    grids = [g for (nm, g) in groups if kernel_key(nm) == kernel_key(name)]
    if kernel_key(name) == "decode_kernel":
        return grid == min(grids)
    return grid == max(grids)


def counter_sums(d):
    """{kernel key: (sum over its whole-workload dispatches of the counter in KiB,
    dispatches)}, plus {copy: ...}.  The pipelined prefill also launches the
    kernels over segments of the chunks; those dispatches are left out, so the
    figure is per launch over all chunks (as timed for the roofline)."""
    f = find(d, "counter_collection.csv")
    if f is None:
        return {}
    groups = {}
    with open(f) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"]
            if kernel_key(name) is None and "copy" not in name.lower():
                continue
            v, n = groups.get((name, int(r["Grid_Size"])), (0.0, set()))
            n.add(r["Dispatch_Id"])
            groups[(name, int(r["Grid_Size"]))] = (v + float(r["Counter_Value"]), n)
    acc = {}
    for (name, grid), (v, n) in groups.items():
        key = kernel_key(name)
        if key is None:
            key = "copy"
        elif not full_launch(name, grid, groups):
            continue
        v0, n0 = acc.get(key, (0.0, 0))
        acc[key] = (v0 + v, n0 + len(n))
    return acc


def mode_traffic():
    sys.path.insert(0, ROOT)
    import bench

    cmds = []
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rc, d, cmd = launch(["profile_bench.py", "copy"], ["--pmc", counter], f"copy_{counter}", 240)
        cmds.append(cmd)
        if not profiler_ok(rc, d, "counter_collection.csv") or counter_sums(d).get("copy") is None:
            raise SystemExit(f"copy calibration for {counter} failed (exit {rc})")
        rc, d, cmd = launch(BENCH_PMC, ["--pmc", counter, "--kernel-include-regex",
                                        "chain_kr_kernel|intra_kernel|output_kernel|decode_kernel|conv_silu_kernel"],
                            f"bench_{counter}", 600)
        cmds.append(cmd)
        if not profiler_ok(rc, d, "counter_collection.csv"):
            raise SystemExit(f"bench pass for {counter} failed (exit {rc})")
    # the kernel sources these counters belong to
    with open(os.path.join(OUT, "traffic_meta.json"), "w") as f:
        json.dump({"sources_digest": bench.kernel_sources_digest(), "commands": cmds}, f, indent=1)
    summarize_traffic()


def summarize_traffic():
    """traffic.json in the output directory, from the raw counter passes."""
    with open(os.path.join(OUT, "traffic_meta.json")) as f:
        meta = json.load(f)
    result = {"sources_digest": meta["sources_digest"], "counters": {}, "calibration": {}, "kernels": {}}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        kib, n = counter_sums(os.path.join(OUT, f"copy_{counter}"))["copy"]
        factor = COPY_BYTES / (kib * 1024.0 / n)
        result["calibration"][counter] = {"copy_bytes": COPY_BYTES, "counted_KiB_per_dispatch": kib / n,
                                          "factor": factor}
        for key, (kib, n) in counter_sums(os.path.join(OUT, f"bench_{counter}")).items():
            if key == "copy":
                continue
            result["counters"].setdefault(key, {})[counter] = {"KiB_per_dispatch": kib / n, "dispatches": n}
    for key, ent in result["counters"].items():
        fetch = ent["FETCH_SIZE"]["KiB_per_dispatch"] * 1024 * result["calibration"]["FETCH_SIZE"]["factor"]
        write = ent["WRITE_SIZE"]["KiB_per_dispatch"] * 1024 * result["calibration"]["WRITE_SIZE"]["factor"]
        result["kernels"][key] = {"fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
                                  "hbm_bytes_per_launch": fetch + write}
    result["commands"] = meta["commands"]
    with open(os.path.join(OUT, "traffic.json"), "w") as f:
        json.dump(result, f, indent=1)
    log(f"[profile] wrote {os.path.join(OUT, 'traffic.json')}")


def render_traffic():
    if os.path.exists(os.path.join(OUT, "traffic_meta.json")):
        summarize_traffic()
    p = os.path.join(OUT, "traffic.json")
    if not os.path.exists(p):
        log("[profile] no traffic output to render")
        return
    with open(p) as f:
        result = json.load(f)
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(result, f, indent=1)
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)", "",
             "Commands (repository root, one MI355X), one counter per pass:", "", "```", *result["commands"], "```", "",
             "Calibration (a device copy of 1 GiB): "
             + ", ".join(f"{c} factor {v['factor']:.3f}" for c, v in result["calibration"].items()), "",
             "Per launch over the whole workload (the pipelined prefill's launches over",
             "segments of the chunks are left out).", "",
             "| kernel | fetch MB/launch | write MB/launch | total MB/launch |", "|---|---|---|---|"]
    for key, ent in sorted(result["kernels"].items()):
        lines.append(f"| `{key}` | {ent['fetch_bytes_per_launch'] / 1e6:.1f} | {ent['write_bytes_per_launch'] / 1e6:.1f}"
                     f" | {ent['hbm_bytes_per_launch'] / 1e6:.1f} |")
    lines += ["", f"Kernel sources digest: `{result['sources_digest']}`", ""]
    with open(os.path.join(PROFILES, "traffic_prefill64k_decode.md"), "w") as f:
        f.write("\n".join(lines))
    log("[profile] wrote profiles/traffic.json and profiles/traffic_prefill64k_decode.md")


MFMA_COUNTERS = ("MfmaUtil", "MfmaFlops", "MfmaFlopsBF16", "MfmaFlopsF32")
MFMA_KERNELS = "chain_kr_kernel|intra_kernel|output_kernel"
BENCH_PMC_BWD = ["bench.py", "--steps", "1", "--warmup", "1", "--no-decode", "--no-other", "--no-cpu-baseline"]


def mode_mfma():
    passes = ((BENCH_PMC, MFMA_KERNELS, "mfma"), (BENCH_PMC_BWD, "bwd_local_kernel|bwd_chain_kernel|bwd_grad_kernel",
                                                   "mfma_bwd"))
    for bench_cmd, regex, tag in passes:
        rc, d, cmd = launch(bench_cmd, ["--pmc", *MFMA_COUNTERS, "--kernel-include-regex", regex], tag, 600)
        with open(os.path.join(d, "command.txt"), "w") as f:
            f.write(cmd + "\n")
        if not profiler_ok(rc, d, "counter_collection.csv"):
            raise SystemExit(f"{tag} pass failed (exit {rc})")


def mfma_table(d):
    """{kernel key: {counter: mean per whole-workload dispatch, "ns": mean duration, "n": dispatches}}."""
    f = find(d, "counter_collection.csv")
    if f is None:
        return {}
    per = {}  # (name, grid) -> {dispatch: {counter: value, "ns": duration}}
    with open(f) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"]
            if kernel_key(name) is None:
                continue
            disp = per.setdefault((name, int(r["Grid_Size"])), {}).setdefault(r["Dispatch_Id"], {})
            disp[r["Counter_Name"]] = disp.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            disp["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            disp["wg"] = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
    out = {}
    for (name, grid), disps in per.items():
        if not full_launch(name, grid, per):
            continue
        key = kernel_key(name)
        n = len(disps)
        ent = {c: sum(v.get(c, 0.0) for v in disps.values()) / n for c in (*MFMA_COUNTERS, "ns", "wg")}
        if key in out:  # several whole-workload instances (the backward chain per d_k): keep the first
            continue
        ent["n"] = n
        out[key] = ent
    return out


def render_mfma():
    d = os.path.join(OUT, "mfma")
    table = mfma_table(d)
    if not table:
        log("[profile] no mfma output to render")
        return
    sys.path.insert(0, ROOT)
    import bench

    chain_alg = bench.flops_chain_per_token() * bench.T
    cmd = open(os.path.join(d, "command.txt")).read().strip()
    lines = ["# MFMA work per launch: 64K-token prefill (H=6, d=256, bf16)", "",
             "Command (repository root, one MI355X), one counter pass:", "", "```", cmd, "```", "",
             "Per launch over the whole workload (the pipelined prefill's launches over",
             "segments of the chunks are left out).  `MfmaFlops` counts the matrix flops",
             "the hardware executed, fp32 operands split into bf16 parts included;",
             "`MfmaUtil` is the MFMA units' busy share over all 1024 SIMDs of the chip for",
             "the dispatch's duration (the dispatch runs alone while counters are taken);",
             "the last column rescales it to the CUs the working workgroups occupy (one",
             "per CU when there are fewer than the chip's 256 CUs; the chain's grid is",
             "padded to whole groups of 8 (sequence, head) pairs, and the padding's",
             "workgroups return at once, so 6 heads x 16 row blocks = 96 work).", "",
             "| kernel | dispatches | workgroups | us (counter run) | executed GFLOP | of which bf16"
             " | executed TFLOP/s | MfmaUtil % | % per occupied CU |", "|---|---|---|---|---|---|---|---|---|"]
    for key in ("intra_kernel", "chain_kr_kernel", "output_kernel"):
        e = table.get(key)
        if e is None:
            continue
        tf = e["MfmaFlops"] / (e["ns"] * 1e-9) / 1e12 if e["ns"] > 0 else float("nan")
        working = bench.H * (bench.DV // 16) if key == "chain_kr_kernel" else e["wg"]
        occ = e["MfmaUtil"] * 256 / min(256.0, max(1.0, working))
        lines.append(f"| `{key}` | {e['n']} | {e['wg']:.0f} | {e['ns'] / 1e3:.0f} | {e['MfmaFlops'] / 1e9:.1f}"
                     f" | {e['MfmaFlopsBF16'] / 1e9:.1f} | {tf:.1f} | {e['MfmaUtil']:.2f} | {occ:.2f} |")
    ch = table.get("chain_kr_kernel")
    if ch is not None:
        lines += ["", f"State chain: algorithmic {chain_alg / 1e9:.1f} GFLOP per launch (4 d_k d_v per token and head);",
                  f"executed / algorithmic = {ch['MfmaFlops'] / chain_alg:.2f}.", ""]
    bwd = mfma_table(os.path.join(OUT, "mfma_bwd"))
    if bwd:
        bcmd = open(os.path.join(OUT, "mfma_bwd", "command.txt")).read().strip()
        alg = bench.flops_backward_per_token() * bench.T
        lines += ["", "## Backward of the same prefill (fp32)", "", "```", bcmd, "```", "",
                  "| kernel | dispatches | workgroups | us (counter run) | executed GFLOP | of which fp32"
                  " | executed TFLOP/s | MfmaUtil % |", "|---|---|---|---|---|---|---|---|"]
        total = 0.0
        for key in ("bwd_local_kernel", "bwd_chain_kernel", "bwd_grad_kernel"):
            e = bwd.get(key)
            if e is None:
                continue
            total += e["MfmaFlops"]
            tf = e["MfmaFlops"] / (e["ns"] * 1e-9) / 1e12 if e["ns"] > 0 else float("nan")
            lines.append(f"| `{key}` | {e['n']} | {e['wg']:.0f} | {e['ns'] / 1e3:.0f} | {e['MfmaFlops'] / 1e9:.1f}"
                         f" | {e['MfmaFlopsF32'] / 1e9:.1f} | {tf:.1f} | {e['MfmaUtil']:.2f} |")
        lines += ["", f"Algorithmic {alg / 1e9:.1f} GFLOP per backward (bench.py's count);",
                  f"executed on MFMA / algorithmic = {total / alg:.2f}.  The executed figure leaves out the",
                  "vector-ALU work (forward substitution, reductions, norms) and counts the",
                  "triangular products as full 64 x 64 blocks.", ""]
    with open(os.path.join(PROFILES, "mfma_prefill64k.md"), "w") as f:
        f.write("\n".join(lines))
    log("[profile] wrote profiles/mfma_prefill64k.md")


def mode_render():
    render_trace()
    render_traffic()
    render_mfma()


def mode_copy():
    import torch

    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")  # no fill: the copy is the only kernel
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print("copied", COPY_BYTES, "bytes", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--out" in args:
        i = args.index("--out")
        OUT = os.path.abspath(args[i + 1])
        del args[i:i + 2]
    mode = args[0] if args else "trace"
    {"trace": mode_trace, "traffic": mode_traffic, "mfma": mode_mfma, "render": mode_render,
     "copy": mode_copy}[mode]()
