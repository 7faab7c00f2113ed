"""Collect and summarize rocprofv3 measurements of the kernels.

    python -m param_collectives_amd.profiling trace    --workload W --out DIR
    python -m param_collectives_amd.profiling counters --workload W --out DIR
    python -m param_collectives_amd.profiling summarize --workload W --out DIR --profiles profiles/

`trace` runs bench.py under `rocprofv3 --kernel-trace --stats` twice: the
timed step and the copy-in (with the sections whose reduce-scatter launches
share the timed kernel's name left out), then the stock path alone (W stock
packs and the fp32 reduce-scatter of the packed buffers); `counters` runs one
`rocprofv3 --pmc` pass per counter group (a group never exceeds one hardware
block's counter slots) on single-kernel launches of bench.py, and on
PyTorch's own fill and neg kernels over buffers of known size; `summarize`
reads those outputs and writes short text summaries and
profiles/hbm_traffic.json.

HBM traffic, two independent ways:
  * FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
    known bytes to counted bytes for a plain stream of known size outside this
    library (PyTorch's elementwise neg, one bf16 read and one write per
    element); this is the `traffic` figure the benchmark reports;
  * the L2-to-memory requests that went to DRAM, counted in 32-byte units
    (TCC_EA0_RDREQ_DRAM_32B, TCC_EA0_WRREQ_WRITE_DRAM_32B): bytes with no
    calibration factor.
On gfx950 the FETCH_SIZE expression takes its 128-byte reads from TCC_BUBBLE,
which stays 0 while every streaming read goes out as a 128-byte request, so
FETCH_SIZE reads half the bytes; the calibration factor is that 2.
A third pass counts the cycles the L2 waited for DRAM credits and the reads
in flight (for the mean read latency).  Every figure is tied to the SHA-256 of
the kernel source, so that a stale one is never reported.  rocprofv3 is
always started as a child process with the program to profile directly after
`--`.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import sqlite3
import statistics
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_SOURCES = [os.path.join(HERE, "csrc", n) for n in ("kernels.hip", "plan.cpp")]
KERNEL_REGEX = "rs_local_kernel|ag_copyout_kernel|ag_copyin_kernel|stock_pack_kernel"
# PyTorch's fill and neg kernels (bench.py --only torch): the calibration streams
TORCH_REGEX = "FillFunctor|neg_kernel"
KERNELS = ("rs_local_kernel", "ag_copyout_kernel", "ag_copyin_kernel", "stock_pack_kernel")
COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "dram": ["TCC_EA0_RDREQ_DRAM_32B", "TCC_EA0_WRREQ_WRITE_DRAM_32B"],
    "stall": ["TCC_EA0_RDREQ_DRAM_CREDIT_STALL", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL", "TCC_EA0_RDREQ_LEVEL",
              "TCC_EA0_RDREQ", "GRBM_GUI_ACTIVE"],
}
COUNTER_MODES = ("rs", "co", "ci", "stock", "torch")
# L2 channels per XCD and XCDs: the TCC counters are summed over all 128
# channels, GRBM_GUI_ACTIVE over the 8 XCDs
TCC_CHANNELS = 16 * 8
XCDS = 8


def _portable(cmd_text, out_root=None):
    """A recorded command with this checkout's absolute paths replaced by
    placeholders: <repo> for the repository root, <out> for the output folder."""
    text = cmd_text
    if out_root:
        text = text.replace(out_root, "<out>")
    text = text.replace(ROOT + "/", "<repo>/").replace(sys.executable, "python")
    return text


def source_digest():
    """SHA-256 over the sources that decide the kernels' memory traffic: the
    kernels and the planner that lays out their segments and vector bodies."""
    h = hashlib.sha256()
    for path in TRAFFIC_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _run(cmd, log):
    print("+", " ".join(shlex.quote(c) for c in cmd), flush=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    with open(log, "w") as f:
        rc = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, cwd="/tmp", env=env, timeout=600).returncode
    print(f"  exit {rc} (log {log})", flush=True)
    if rc != 0:
        raise SystemExit(rc)


def bench_cmd(workload, extra):
    return [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, *extra]


TRACE_STEPS = 10
COUNTER_LAUNCHES = 3


def trace_op_calls(run, kernel, world):
    """Operation calls each trace run makes of a kernel (bench.py: warm-up 2 +
    timed steps of the reduce-scatter and copy-out, three untimed + 10 timed
    copy-ins; the stock run: W packs and one reduce per launch).  An operation
    call may be several dispatches (long operations are split)."""
    calls = {("trace", "rs_local_kernel"): TRACE_STEPS + 2, ("trace", "ag_copyout_kernel"): TRACE_STEPS + 2,
             ("trace", "ag_copyin_kernel"): 13, ("trace_stock", "stock_pack_kernel"): TRACE_STEPS * world,
             ("trace_stock", "rs_local_kernel"): TRACE_STEPS}
    return calls.get((run, kernel))


def collect_trace(workload, out, steps=TRACE_STEPS):
    os.makedirs(out, exist_ok=True)
    runs = {"trace": ["--steps", str(steps), "--warmup", "2", "--no-cpu-baseline", "--no-sweep", "--no-extras"],
            "trace_stock": ["--only", "stock", "--launches", str(steps)]}
    for name, extra in runs.items():
        cmd = ["rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d", os.path.join(out, name), "-o", name,
               "--", *bench_cmd(workload, extra)]
        _run(cmd, os.path.join(out, name + ".log"))
        with open(os.path.join(out, name + ".cmd"), "w") as f:
            f.write(_portable(" ".join(shlex.quote(c) for c in cmd), out) + "\n")


def collect_counters(workload, out, launches=COUNTER_LAUNCHES):
    os.makedirs(out, exist_ok=True)
    cmds = {}
    for only in COUNTER_MODES:
        for name, counters in COUNTER_PASSES.items():
            d = os.path.join(out, f"pmc_{only}_{name}")
            regex = TORCH_REGEX if only == "torch" else KERNEL_REGEX
            cmd = ["rocprofv3", "--pmc", *counters, "--kernel-include-regex", regex, "-f", "csv", "-d", d,
                   "-o", "pmc", "--", *bench_cmd(workload, ["--only", only, "--launches", str(launches)])]
            _run(cmd, d + ".log")
            cmds[f"{only}_{name}"] = _portable(" ".join(shlex.quote(c) for c in cmd), out)
    with open(os.path.join(out, "counters.cmd.json"), "w") as f:
        json.dump(cmds, f, indent=1)


def _normalise(text):
    """Commands recorded on another machine: keep only repo-relative parts."""
    import re

    text = re.sub(r"-d \S*/([^/ ]+)(?= )", r"-d <out>/\1", text)
    text = re.sub(r"\S*/bench\.py", "<repo>/bench.py", text)
    text = re.sub(r"\S*/python3?(?= )", "python", text)
    return text


def _read_counter(d, counter):
    """Per-dispatch values of one counter, summed over its instances."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    names = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = r["Dispatch_Id"]
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                names[key] = r["Kernel_Name"]
    return [(names[k], v) for k, v in sorted(per.items(), key=lambda kv: int(kv[0]))]


def _short(name):
    for k in KERNELS:
        if k in name:
            return k
    return name[:60]


def _kernel_stats(out, run="trace"):
    files = glob.glob(os.path.join(out, run, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    if rows:
        return rows
    dbs = glob.glob(os.path.join(out, run, "**", "*.db"), recursive=True)
    for db in dbs:
        con = sqlite3.connect(db)
        for name, calls, total, avg, pct in con.execute("select name, total_calls, total_duration, average, percentage "
                                                        "from top_kernels"):
            rows.append({"Name": name, "Calls": calls, "TotalDurationNs": total, "AverageNs": avg, "Percentage": pct})
    return rows


def _kernel_trace_rows(out, run="trace"):
    """(kernel short name, duration in ns) of every dispatch of a trace run,
    in dispatch order."""
    rows = []
    for fn in glob.glob(os.path.join(out, run, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                rows.append((int(r.get("Dispatch_Id", 0) or 0), _short(r.get("Kernel_Name", "")),
                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    return [(name, ns) for _, name, ns in rows]


def _launch_bytes(plan, op, W):
    """Algorithmic bytes of each launch of one call of `op` (0 reduce-scatter,
    1 copy-out, 2 copy-in), from the segment table and the launch table:
    a summed element moves 2W bytes in and 4 out, a padding element of a shard
    4 out; a copied element 2 + 2 (copy-out) or 4 + 2 (copy-in from fp32), a
    padding slot of the rank-major buffer 2 out."""
    import numpy as np

    segs = plan.segments(op)
    chunk = plan.options(op)["chunk_elems"]
    nch = -(-segs[:, 5] // chunk)
    first = np.concatenate([[0], np.cumsum(nch)])
    per_kind = {0: {0: 2 * W + 4, 1: 4}, 1: {2: 4}, 2: {2: 6, 1: 2}}[op]
    out = []
    for c0, c1, s0, s1, _ in plan.launches(op, cu_count=256):
        b = 0
        for i in range(s0, s1):
            lo, hi = max(c0, first[i]), min(c1, first[i + 1])
            if hi > lo:
                e = min((hi - first[i]) * chunk, segs[i, 5]) - (lo - first[i]) * chunk
                b += int(e) * per_kind[int(segs[i, 0])]
        out.append(b)
    return out


def _per_launch_lines(out, workload):
    """Per launch position within a call of the timed step's kernels: the
    median duration over the run's calls (the first left out) and the rate."""
    import numpy as np

    import synth
    from param_collectives_amd import tide

    w = synth.workload(workload)
    plan = tide.Plan(w.world, w.shapes)
    rows = _kernel_trace_rows(out)
    lines = []
    for op, kernel in ((0, "rs_local_kernel"), (1, "ag_copyout_kernel"), (2, "ag_copyin_kernel")):
        ns = [d for name, d in rows if name == kernel]
        nbytes = _launch_bytes(plan, op, w.world)
        n = len(nbytes)
        if not ns or len(ns) % n:
            continue
        calls = np.array(ns, dtype=np.float64).reshape(-1, n)[1:]
        med = np.median(calls, axis=0) / 1e3
        lines.append(f"{kernel}: {n} launches per call (chunks of each launch: tide_plan_launches), "
                     f"median of {len(calls)} calls")
        lines.append("  " + " ".join(f"{i}:{m:.1f}us/{b / m / 1e6:.2f}TB/s" for i, (m, b) in
                                     enumerate(zip(med, nbytes))))
    return lines


def summarize(workload, out, profiles):
    os.makedirs(profiles, exist_ok=True)
    digest = source_digest()
    # kernel traces: the timed step (+ copy-in), then the stock path alone,
    # whose reduce-scatter is the fp32 instance of rs_local_kernel
    lines = [f"# rocprofv3 kernel trace: {workload}", "", f"kernels.hip + plan.cpp sha256: {digest}"]
    any_stats = False
    for run, title in (("trace", "timed step (reduce-scatter from bf16 gradients, copy-out) and copy-in"),
                       ("trace_stock", "stock path: W stock packs, then the reduce-scatter of the W packed fp32 "
                                       "buffers (rs_local_kernel here is its fp32-source instance)")):
        stats = _kernel_stats(out, run)
        if not stats:
            continue
        any_stats = True
        lines += ["", f"## {title}"]
        try:
            lines.append("command (run in /tmp): " + _normalise(open(os.path.join(out, run + ".cmd")).read().strip()))
        except OSError:
            pass
        lines.append("per dispatch (avg, min, max) and per operation call (all dispatches of one call; long "
                     "operations are split into several dispatches)")
        lines.append(f"{'kernel':<22} {'dispatches':>10} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6} "
                     f"{'op_calls':>8} {'us_per_call':>12}")
        import synth

        world = synth.workload(workload).world
        for r in stats:
            name = _short(r.get("Name", r.get("KernelName", "")))
            if name not in KERNELS:
                continue
            avg = float(r.get("AverageNs", 0)) / 1e3
            mn = float(r.get("MinNs", 0) or 0) / 1e3
            mx = float(r.get("MaxNs", 0) or 0) / 1e3
            calls = trace_op_calls(run, name, world)
            per_call = float(r.get("TotalDurationNs", 0)) / 1e3 / calls if calls else float("nan")
            lines.append(f"{name:<22} {r.get('Calls', ''):>10} {avg:>10.2f} {mn:>10.2f} {mx:>10.2f} "
                         f"{float(r.get('Percentage', 0)):>6.1f} {calls!s:>8} {per_call:>12.2f}")
    if any_stats:
        per_launch = _per_launch_lines(out, workload)
        if per_launch:
            lines += ["", "## timed step, per launch within a call (launch index: median duration / rate)"]
            lines += per_launch
        with open(os.path.join(profiles, f"kernel_trace_{workload}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # counters
    cdir = out
    if not os.path.isdir(os.path.join(cdir, "pmc_torch_fetch")):
        return
    cmds = {k: _normalise(v) for k, v in json.load(open(os.path.join(cdir, "counters.cmd.json"))).items()}

    def total(only, name, counter, kernel, calls=COUNTER_LAUNCHES):
        """One operation call's worth of a counter: summed over every
        dispatch of the kernel, divided by the operation calls made."""
        vals = [v for n, v in _read_counter(os.path.join(cdir, f"pmc_{only}_{name}"), counter) if kernel in n]
        return sum(vals) / calls if vals else None

    import synth
    from param_collectives_amd import tide

    w = synth.workload(workload)
    W = w.world
    plan = tide.Plan(W, w.shapes)
    sum_dk = sum(plan.numel)
    S = plan.shard_elems
    known = 2 * W * S  # bytes each calibration stream reads and/or writes
    nf, nw = total("torch", "fetch", "FETCH_SIZE", "neg_kernel"), total("torch", "write", "WRITE_SIZE", "neg_kernel")
    cal = {"kernel": "PyTorch's elementwise neg over W*S bf16 (one read and one write per element)",
           "bytes_read": known, "bytes_written": known, "fetch_kib": nf, "write_kib": nw,
           "fetch_factor": known / (nf * 1024.0), "write_factor": known / (nw * 1024.0)}
    checks = {}
    for label, kern, alg_r, alg_w in (("torch_neg", "neg_kernel", known, known),
                                      ("torch_fill", "FillFunctor", 0, known)):
        rd = total("torch", "dram", "TCC_EA0_RDREQ_DRAM_32B", kern)
        wd = total("torch", "dram", "TCC_EA0_WRREQ_WRITE_DRAM_32B", kern)
        if rd is not None and wd is not None:
            checks[label] = {"dram_read_bytes": 32.0 * rd, "dram_write_bytes": 32.0 * wd,
                             "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w}
    kernels = {}
    for only, kname, key, alg_r, alg_w in (("rs", "rs_local", "rs_local", 2 * W * sum_dk, 4 * W * S),
                                           ("co", "ag_copyout", "ag_copyout", 2 * sum_dk, 2 * sum_dk),
                                           ("ci", "ag_copyin", "ag_copyin", 4 * sum_dk, 2 * W * S),
                                           ("stock", "stock_pack", "stock_pack", 2 * sum_dk, 4 * W * S),
                                           ("stock", "rs_local", "rs_local_f32_packed", 4 * W * W * S, 4 * W * S)):
        kname = kname + "_kernel"
        if not os.path.isdir(os.path.join(cdir, f"pmc_{only}_fetch")):
            continue
        calls = COUNTER_LAUNCHES * (W if kname == "stock_pack_kernel" else 1)
        f = total(only, "fetch", "FETCH_SIZE", kname, calls)
        wr = total(only, "write", "WRITE_SIZE", kname, calls)
        if f is None or wr is None:
            continue
        traffic_r = f * 1024.0 * cal["fetch_factor"]
        traffic_w = wr * 1024.0 * cal["write_factor"]
        k = {"fetch_kib": f, "write_kib": wr, "hbm_read_bytes": traffic_r, "hbm_write_bytes": traffic_w,
             "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w,
             "read_ratio": traffic_r / alg_r, "write_ratio": traffic_w / alg_w}
        rd = total(only, "dram", "TCC_EA0_RDREQ_DRAM_32B", kname, calls)
        wd = total(only, "dram", "TCC_EA0_WRREQ_WRITE_DRAM_32B", kname, calls)
        if rd is not None and wd is not None:
            k.update({"dram_read_bytes": 32.0 * rd, "dram_write_bytes": 32.0 * wd,
                      "dram_read_ratio": 32.0 * rd / alg_r, "dram_write_ratio": 32.0 * wd / alg_w})
        st = {c: total(only, "stall", c, kname, calls) for c in COUNTER_PASSES["stall"]}
        if all(v is not None for v in st.values()) and st["GRBM_GUI_ACTIVE"]:
            cycles = st["GRBM_GUI_ACTIVE"] / XCDS  # per XCD, over the call
            k.update({
                "busy_cycles": cycles,
                "read_credit_stall_frac": st["TCC_EA0_RDREQ_DRAM_CREDIT_STALL"] / (TCC_CHANNELS * cycles),
                "write_credit_stall_frac": st["TCC_EA0_WRREQ_DRAM_CREDIT_STALL"] / (TCC_CHANNELS * cycles),
                "read_latency_cycles": st["TCC_EA0_RDREQ_LEVEL"] / st["TCC_EA0_RDREQ"],
                "reads_in_flight": st["TCC_EA0_RDREQ_LEVEL"] / cycles})
        kernels[f"{key}/{workload}"] = k
    path = os.path.join(profiles, "hbm_traffic.json")
    try:
        t = json.load(open(path))
        if t.get("source_sha256") != digest:
            t = {}
    except (OSError, ValueError):
        t = {}
    t["source_sha256"] = digest
    t["calibration"] = cal
    t.setdefault("calibration_checks", {}).update({f"{k}/{workload}": v for k, v in checks.items()})
    t.setdefault("kernels", {}).update(kernels)
    t.setdefault("commands", {})[workload] = cmds
    with open(path, "w") as fo:
        json.dump(t, fo, indent=1, sort_keys=True)
    txt = [f"# HBM traffic per operation call from rocprofv3 counters: {workload}", "",
           f"kernels.hip + plan.cpp sha256: {digest}", "",
           "calibration (a plain stream of known size outside this library: PyTorch's elementwise neg):",
           f"  {known} B each way; FETCH_SIZE {nf:.0f} KiB, WRITE_SIZE {nw:.0f} KiB;"
           f" factors read {cal['fetch_factor']:.4f}, write {cal['write_factor']:.4f}"]
    for label, v in checks.items():
        txt.append(f"  {label}: DRAM read {v['dram_read_bytes'] / 1e9:.4f} GB, DRAM write "
                   f"{v['dram_write_bytes'] / 1e9:.4f} GB (known: {v['algorithmic_read_bytes'] / 1e9:.4f} GB read, "
                   f"{v['algorithmic_write_bytes'] / 1e9:.4f} GB written)")
    txt += ["", "per kernel: FETCH_SIZE/WRITE_SIZE scaled by the factors | DRAM bytes from the 32-byte request "
                "counters (no factor) | cycles waiting for DRAM credits (read, write; fraction of L2-channel "
                "cycles) | mean read latency (cycles) and reads in flight"]
    for k, v in kernels.items():
        line = (f"{k}: read {v['hbm_read_bytes'] / 1e9:.4f} GB ({v['read_ratio']:.3f} x algorithmic), "
                f"write {v['hbm_write_bytes'] / 1e9:.4f} GB ({v['write_ratio']:.3f} x)")
        if "dram_read_bytes" in v:
            line += (f" | DRAM read {v['dram_read_bytes'] / 1e9:.4f} GB ({v['dram_read_ratio']:.4f} x), "
                     f"write {v['dram_write_bytes'] / 1e9:.4f} GB ({v['dram_write_ratio']:.4f} x)")
        if "read_latency_cycles" in v:
            line += (f" | credit stalls {v['read_credit_stall_frac']:.3f}, {v['write_credit_stall_frac']:.3f}"
                     f" | read latency {v['read_latency_cycles']:.0f}, in flight {v['reads_in_flight']:.0f}")
        txt.append(line)
    txt += ["", "commands (each run in /tmp; <repo> is the repository root, <out> the output folder):"]
    txt += [f"  {k}: {c}" for k, c in sorted(cmds.items())]
    with open(os.path.join(profiles, f"hbm_traffic_{workload}.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("action", choices=["trace", "counters", "summarize"])
    ap.add_argument("--workload", default="llama3.1-8b-layer")
    ap.add_argument("--out", required=True)
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    out = os.path.abspath(args.out)
    if args.action == "trace":
        collect_trace(args.workload, out)
    elif args.action == "counters":
        collect_counters(args.workload, out)
    else:
        summarize(args.workload, out, args.profiles)


if __name__ == "__main__":
    main()
