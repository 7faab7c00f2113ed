#!/usr/bin/env python3
"""Benchmark of the layout-aware FSDP2 collective local stages on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the reduce-scatter local stage (W ranks' bf16
gradients -> W packed fp32 shards) followed by the all-gather copy-out
(rank-major bf16 buffer -> per-parameter tensors), on one HIP stream.  The
shard-layout plan is made once, before timing (it is per-registration work).

Reported (one JSON line): effective HBM GB/s of the step, i.e. algorithmic
bytes read plus written by the step's two operations divided by the step
time, with
  * the all-gather copy-in (fp32 master shards -> rank-major bf16, fused
    cast) timed beside the step, not part of it;
  * per-kernel figures from HIP events recorded on the kernels' own stream;
  * the roofline of the dominant kernel (the reduce-scatter) against MI355X's
    8 TB/s HBM peak, and its measured HBM traffic when a counter summary for
    the current kernel source is committed under profiles/;
  * a CU-budget sweep, each kernel on a stream masked to the budget's CUs,
    with one and with four workgroups per CU (GB/s per CU is the analog of
    the pages' per-CTA sum rate);
  * a plain device-to-device copy of the copy-out's byte count, and the
    copy-out kernel on one flat tensor of the same bytes, for context;
  * Equation 5's epilogue (alpha = 1/W, accumulate into the shards) and the
    reduce-scatter from fp32 gradients, per kernel;
  * the stock path A/B: W stock gradient packs (slice, zero-pad, widen, pack
    rank-major into W*S fp32 per rank) followed by the fp32 reduce-scatter
    of the packed buffers, against the layout-aware reduce-scatter that
    replaces both (same shards, bit for bit, checked in the run);
  * the CPU oracle timed on the host's cores on the same workload, streamed
    in groups of parameters so that host memory stays bounded, with a
    bitwise check of the run's outputs against it.
Algorithmic bytes: reduce-scatter 2*W*sum(D*K) read + 4*W*S written (padding
is written, never read); copy-out 2*sum(D*K) read + 2*sum(D*K) written.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "effective HBM GB/s (and % of peak) for RS-local reduce and AG copy-out"
DEFAULT_WORKLOAD = "llama3.1-70b-layer"
# host memory the CPU leg holds at once: one group of parameters' gradients
GROUP_BYTES = 8_000_000_000
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
TRAFFIC_SOURCES = [os.path.join(ROOT, "param_collectives_amd", "csrc", n) for n in ("kernels.hip", "plan.cpp")]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--world", type=int, default=0,
                    help="simulated ranks W, overriding the workload's (same shapes; 0 = the workload's own)")
    ap.add_argument("--cu-budget", type=int, default=0)
    ap.add_argument("--wg-per-cu", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--wave-chunks", type=int, default=0, help="chunks per wave per launch (0 = default)")
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true", help="skip the CU-budget sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work the oracle leg repeats its steps for (at least 3 per parameter group)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the Equation 5 epilogue, stock-path A/B and flat-copy sections (their launches "
                         "share the kernel names of the timed ones)")
    ap.add_argument("--only", choices=["rs", "co", "ci", "calib", "stock", "torch"],
                    help="launch just one kernel (stock: the W packs and the fp32 reduce-scatter of the stock "
                         "path; torch: PyTorch's own fill and neg kernels over W*S bf16 elements, plain "
                         "streams of known size for calibrating counters) --launches times, for profiling, and "
                         "exit")
    ap.add_argument("--launches", type=int, default=5)
    return ap.parse_args(argv)


def source_digest():
    """SHA-256 over the sources that decide the kernels' memory traffic: the
    kernels and the planner that lays out their segments and vector bodies."""
    h = hashlib.sha256()
    for path in TRAFFIC_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(kernel_key):
    """HBM bytes per operation call from the committed counter summary:
    (FETCH_SIZE + WRITE_SIZE scaled by a plain stream's calibration factors,
    DRAM bytes from the 32-byte request counters), or (None, None) when there
    is none for this kernel and workload or the kernel source changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("source_sha256") != source_digest():
        return None, None
    k = t.get("kernels", {}).get(kernel_key)
    cal = t.get("calibration")
    if not k or not cal:
        return None, None
    scaled = k["fetch_kib"] * 1024.0 * cal["fetch_factor"] + k["write_kib"] * 1024.0 * cal["write_factor"]
    dram = k["dram_read_bytes"] + k["dram_write_bytes"] if "dram_read_bytes" in k else None
    return scaled, dram


def cpu_model():
    """The host CPU's model name and the cores visible to this process."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name}; {len(os.sched_getaffinity(0))} cores visible"


def launches_per_call(plan, op):
    """Kernel launches one call of operation `op` makes (the library's own
    split: at most wave_chunks chunks per wave per launch)."""
    return len(plan.launches(op))


def param_groups(w, max_bytes):
    """Consecutive parameters grouped so that one group's W ranks' bf16
    gradients take at most max_bytes of host memory (a larger parameter is a
    group of its own)."""
    groups, cur, cur_bytes = [], [], 0
    for p in range(w.nparams):
        b = 2 * w.world * w.numel(p)
        if cur and cur_bytes + b > max_bytes:
            groups.append(cur)
            cur, cur_bytes = [], 0
        cur.append(p)
        cur_bytes += b
    if cur:
        groups.append(cur)
    return groups


def cpu_leg(w, plan, grads, outs, rank_major, params, step_bytes, budget_s):
    """The CPU oracle timed on the host's cores on the same workload, and the
    bitwise verdict of this run's GPU outputs against it.

    Host memory stays bounded: the parameters are taken in consecutive groups
    of at most GROUP_BYTES of gradients.  A group's parameters occupy one
    contiguous range of every rank's shard and of every rank-major slot, so
    the oracle run on the group's shapes alone yields exactly those ranges.
    Each group's oracle step (reduce-scatter, then copy-out) is repeated for
    its share of `budget_s`; the step time is the sum over groups of the
    median repetition, and one repetition on a single thread must give the
    same bits."""
    import numpy as np
    import torch

    import oracle

    W, S = w.world, plan.shard_elems
    threads = min(16, len(os.sched_getaffinity(0)))
    total_elems = sum(w.numel(p) for p in range(w.nparams))
    med_sum = one_sum = spent = 0.0
    reps_total = 0
    ok = ok_co = same_threads = True
    groups = param_groups(w, GROUP_BYTES)
    rm2d = rank_major.view(W, S)
    for grp in groups:
        shapes = [w.shapes[p] for p in grp]
        lo = int(plan.shard_offset[grp[0]])
        hi = int(plan.shard_offset[grp[-1] + 1]) if grp[-1] + 1 < w.nparams else S
        host_g = [[grads[u][p].view(torch.int16).cpu().numpy().view(np.uint16) for p in grp] for u in range(W)]
        host_rm = rm2d[:, lo:hi].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        share = budget_s * sum(w.numel(p) for p in grp) / max(total_elems, 1)
        times = []
        want = want_co = None
        while len(times) < 3 or (sum(times) < share and len(times) < 1000):
            t = time.perf_counter()
            want = oracle.rs_local(W, shapes, host_g, nthreads=threads)
            want_co = oracle.copyout(W, shapes, host_rm, nthreads=threads)
            times.append(time.perf_counter() - t)
        t = time.perf_counter()
        one = oracle.rs_local(W, shapes, host_g, nthreads=1)
        oracle.copyout(W, shapes, host_rm, nthreads=1)
        one_sum += time.perf_counter() - t
        med_sum += statistics.median(times)
        spent += sum(times)
        reps_total += len(times)
        same_threads = same_threads and all(
            np.array_equal(one[r].view(np.uint32), want[r].view(np.uint32)) for r in range(W))
        ok = ok and all(np.array_equal(outs[r][lo:hi].cpu().numpy().view(np.uint32), want[r].view(np.uint32))
                        for r in range(W))
        ok_co = ok_co and all(
            np.array_equal(params[p].view(torch.int16).cpu().numpy().view(np.uint16), want_co[i])
            for i, p in enumerate(grp))
        del host_g, host_rm, want, want_co, one
    cpu = {"value": round(step_bytes / med_sum / 1e9, 2), "unit": "GB/s", "cores": threads,
           "single_thread_value": round(step_bytes / one_sum / 1e9, 2),
           "single_thread_matches": same_threads,
           "kind": "oracle",
           "cpu": cpu_model(),
           "sample": f"every parameter of {w.name} (reduce-scatter + copy-out, same inputs as the GPU), streamed in "
                     f"{len(groups)} groups of at most {GROUP_BYTES / 1e9:.0f} GB of gradients; {reps_total} group "
                     f"steps in {spent:.1f} s; step = sum of the groups' median times, {med_sum:.3f} s; "
                     f"{threads} threads"}
    parity = {"rs_local": "bit-exact" if ok else "MISMATCH", "ag_copyout": "bit-exact" if ok_co else "MISMATCH"}
    return cpu, parity


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: bench.py measures one GPU only (got --gpus {args.gpus}); the W simulated ranks all live "
              "in one GPU's HBM. Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from param_collectives_amd import tide

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    w = synth.workload(args.workload)
    own_world = args.world in (0, w.world)  # the committed counters are for the workload's own W
    if args.world:
        w = dataclasses.replace(w, world=args.world)
    opts = dict(cu_budget=args.cu_budget, wg_per_cu=args.wg_per_cu, chunk_elems=args.chunk, flags=args.flags,
                wave_chunks=args.wave_chunks)
    plan = tide.Plan(w.world, w.shapes, **opts)
    W, S = w.world, plan.shard_elems
    sum_dk = sum(w.numel(p) for p in range(w.nparams))
    rs_bytes = 2 * W * sum_dk + 4 * W * S
    co_bytes = 4 * sum_dk
    stream = torch.cuda.Stream()

    if args.only == "torch":
        # PyTorch's own elementwise kernels over W*S bf16 elements: plain
        # streams of known size, outside this library, for calibrating counters
        n = W * S
        a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        for _ in range(args.launches):
            a.fill_(1.0)  # writes 2n bytes
            torch.neg(a, out=b)  # reads 2n bytes, writes 2n bytes
        torch.cuda.synchronize()
        print(json.dumps({"only": "torch", "launches": args.launches, "fill_bytes_written": 2 * n,
                          "neg_bytes_each_way": 2 * n}))
        return 0

    with torch.cuda.stream(stream):
        grads = synth.grads_device(w, "cuda")
        outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
        rank_major = synth.rank_major_device(w, W * S, "cuda")
        params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in w.shapes]
    stream.synchronize()

    # The buffers are registered once and reused every step, as an FSDP2 group
    # reuses its gradient and parameter storage (pointers marshalled once).
    rs_call = tide.reduce_scatter_call(plan, grads, outs)
    co_call = tide.allgather_copyout_call(plan, rank_major, params)

    def rs():
        rs_call(stream)

    def co():
        co_call(stream)

    def stock_setup():
        """The stock path's buffers and registered calls: W packs of W*S fp32
        and the fp32 reduce-scatter of a (W, S) plan."""
        pack_plan = tide.Plan(W, [(W, S)], **opts)
        with torch.cuda.stream(stream):
            packed = [torch.empty(W * S, dtype=torch.float32, device="cuda") for _ in range(W)]
            stock_outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
        pack_calls = [tide.stock_chunk_cat_call(plan, grads[u], packed[u]) for u in range(W)]
        red_call = tide.reduce_scatter_call(pack_plan, [[t.view(W, S)] for t in packed], stock_outs)
        return pack_calls, red_call, stock_outs

    # every rank: its gradients read, W*S fp32 written; then W packed buffers
    # read and W shards written
    pack_bytes = W * (2 * sum_dk + 4 * W * S)
    red_bytes = 4 * W * W * S + 4 * W * S

    if args.only:
        if args.only == "stock":
            pack_calls, red_call, _ = stock_setup()
            for _ in range(args.launches):
                for c in pack_calls:
                    c(stream)
                red_call(stream)
            stream.synchronize()
            print(json.dumps({"only": "stock", "workload": w.name, "launches": args.launches,
                              "pack_bytes_per_rank": pack_bytes // W, "reduce_bytes": red_bytes}))
        elif args.only == "calib":
            n = W * S
            cplan = tide.Plan(1, [(n,)], **opts)
            dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            for _ in range(args.launches):
                tide.allgather_copyout(cplan, rank_major, [dst], stream=stream)
            stream.synchronize()
            print(json.dumps({"only": "calib", "launches": args.launches, "bytes_read": 2 * n, "bytes_written": 2 * n}))
        elif args.only == "ci":
            gen = torch.Generator(device="cuda")
            gen.manual_seed(synth.device_seed(w.index, 2000))
            masters = [torch.randn(s, generator=gen, device="cuda", dtype=torch.float32) * w.sigma for s in w.shapes]
            shards = [[m[min(r * int(R), s[0]):min((r + 1) * int(R), s[0])]
                       for m, s, R in zip(masters, w.shapes, plan.rows_per_rank)] for r in range(W)]
            for _ in range(args.launches):
                tide.allgather_copyin(plan, shards, rank_major, stream=stream)
            stream.synchronize()
            print(json.dumps({"only": "ci", "workload": w.name, "launches": args.launches,
                              "bytes": 4 * sum_dk + 2 * W * S}))
        else:
            fn = rs if args.only == "rs" else co
            for _ in range(args.launches):
                fn()
            stream.synchronize()
            print(json.dumps({"only": args.only, "workload": w.name, "launches": args.launches,
                              "bytes": rs_bytes if args.only == "rs" else co_bytes}))
        return 0

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # warm-up (also binds the plan and uploads its tables)
    for _ in range(args.warmup):
        rs()
        co()
    stream.synchronize()

    marks = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b, c in marks:
        a.record(stream)
        rs()
        b.record(stream)
        co()
        c.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rs_ms = [a.elapsed_time(b) for a, b, _ in marks]
    co_ms = [b.elapsed_time(c) for _, b, c in marks]
    step_ms_events = marks[0][0].elapsed_time(marks[-1][2]) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    def kstats(ms, nbytes):
        avg = sum(ms) / len(ms)
        med = statistics.median(ms)
        return {"bytes": nbytes, "avg_ms": round(avg, 5), "median_ms": round(med, 5), "min_ms": round(min(ms), 5),
                "p90_ms": round(sorted(ms)[int(0.9 * (len(ms) - 1))], 5), "gbps": round(nbytes / avg / 1e6, 1),
                "frac_of_peak": round(nbytes / avg / 1e6 / HBM_PEAK_GBPS, 4)}

    kernels = {"rs_local": kstats(rs_ms, rs_bytes), "ag_copyout": kstats(co_ms, co_bytes)}

    # the all-gather copy-in (fp32 master shards of every rank -> rank-major
    # bf16, cast fused), measured beside the step: 4*sum(D*K) read, 2*W*S written
    ci_bytes = 4 * sum_dk + 2 * W * S
    with torch.cuda.stream(stream):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(synth.device_seed(w.index, 2000))
        masters = [torch.randn(s, generator=gen, device="cuda", dtype=torch.float32) * w.sigma for s in w.shapes]
        shards = [[m[min(r * int(R), s[0]):min((r + 1) * int(R), s[0])]
                   for m, s, R in zip(masters, w.shapes, plan.rows_per_rank)] for r in range(W)]
        ci_out = torch.empty(W * S, dtype=torch.bfloat16, device="cuda")
        ci_call = tide.allgather_copyin_call(plan, shards, ci_out)
        for _ in range(3):
            ci_call(stream)
        e = [(ev(), ev()) for _ in range(10)]
        for a, b_ in e:
            a.record(stream)
            ci_call(stream)
            b_.record(stream)
    stream.synchronize()
    kernels["ag_copyin_f32"] = kstats([a.elapsed_time(b_) for a, b_ in e], ci_bytes)
    del masters, shards, ci_out, ci_call

    # plain device-to-device copy of the copy-out's byte count (context)
    with torch.cuda.stream(stream):
        src = torch.empty(co_bytes // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        e = [(ev(), ev()) for _ in range(10)]
        for a, b in e:
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
    stream.synchronize()
    d2d_ms = sum(a.elapsed_time(b) for a, b in e) / len(e)
    d2d = {"bytes": co_bytes, "avg_ms": round(d2d_ms, 5), "gbps": round(co_bytes / d2d_ms / 1e6, 1)}
    del src, dst


    def timed(fn, n=10):
        fn()
        e = [(ev(), ev()) for _ in range(n)]
        for a, b in e:
            a.record(stream)
            fn()
            b.record(stream)
        stream.synchronize()
        return [a.elapsed_time(b) for a, b in e]

    def stock_a_b(kstats, kernels):
        """Stock path A/B: W packs then the fp32 reduce-scatter, against the
        layout-aware reduce-scatter (same shards, checked bit for bit)."""
        pack_calls, red_call, stock_outs = stock_setup()
        marks_ab = [(ev(), ev(), ev()) for _ in range(10)]
        for c in pack_calls:
            c(stream)
        red_call(stream)
        for a, b, c_ in marks_ab:
            a.record(stream)
            for c in pack_calls:
                c(stream)
            b.record(stream)
            red_call(stream)
            c_.record(stream)
        stream.synchronize()
        pk_ms = [a.elapsed_time(b) for a, b, _ in marks_ab]
        rd_ms = [b.elapsed_time(c_) for _, b, c_ in marks_ab]
        kernels["stock_pack_xW"] = kstats(pk_ms, pack_bytes)
        kernels["rs_local_f32_packed"] = kstats(rd_ms, red_bytes)
        same = all(torch.equal(stock_outs[r].view(torch.int32), outs[r].view(torch.int32)) for r in range(W))
        stock_ms = kernels["stock_pack_xW"]["avg_ms"] + kernels["rs_local_f32_packed"]["avg_ms"]
        stock_ab = {"stock_ms": round(stock_ms, 5), "layout_aware_ms": kernels["rs_local"]["avg_ms"],
                    "speedup": round(stock_ms / kernels["rs_local"]["avg_ms"], 3),
                    "stock_hbm_bytes": pack_bytes + red_bytes, "layout_aware_hbm_bytes": rs_bytes,
                    "extra_hbm_bytes": pack_bytes + red_bytes - rs_bytes, "extra_buffer_bytes": 4 * W * W * S,
                    "shards": "bit-identical" if same else "MISMATCH"}
        return stock_ab

    def host_enqueue(n=50):
        """Host time to enqueue one operation call, in microseconds: a
        registered call (pointers marshalled once, as an FSDP2 group reuses its
        buffers) and a one-off call (every tensor checked and marshalled)."""
        out = {}
        for name, fn in (
                ("rs_local_registered", rs),
                ("ag_copyout_registered", co),
                ("rs_local_one_off", lambda: tide.reduce_scatter_local(plan, grads, outs, stream=stream)),
                ("ag_copyout_one_off", lambda: tide.allgather_copyout(plan, rank_major, params, stream=stream))):
            fn()
            stream.synchronize()
            t = time.perf_counter()
            for _ in range(n):
                fn()
            dt = time.perf_counter() - t
            stream.synchronize()
            out[name] = round(dt / n * 1e6, 1)
        return out

    stock_ab = None
    host_us = None
    flat = None
    if not args.no_extras:
        # (rewrites the timed outputs with the same values)
        host_us = host_enqueue()
        # Equation 5's epilogue: alpha = 1/W, accumulating into separate shards
        # (the timed outputs stay as they are for the parity check below); the
        # shards are read as well: 4*W*S more bytes
        with torch.cuda.stream(stream):
            acc_outs = [torch.zeros(S, dtype=torch.float32, device="cuda") for _ in range(W)]
        acc_call = tide.reduce_scatter_call(plan, grads, acc_outs, alpha=1.0 / W, accumulate=True)
        kernels["rs_local_alpha_accumulate"] = kstats(timed(lambda: acc_call(stream)), rs_bytes + 4 * W * S)
        del acc_outs, acc_call
        stock_ab = stock_a_b(kstats, kernels)
        # the copy-out kernel on one flat tensor of the same byte count, same
        # launch options: what a plain 1:1 bf16 copy reaches on this GPU, without
        # segment boundaries (context for the copy-out's fraction of peak)
        with torch.cuda.stream(stream):
            fsrc = torch.empty(sum_dk, dtype=torch.bfloat16, device="cuda")
            fdst = torch.empty_like(fsrc)
            fplan = tide.Plan(1, [(sum_dk,)], **opts)
            fcall = tide.allgather_copyout_call(fplan, fsrc, [fdst])
            fcall(stream)
            e = [(ev(), ev()) for _ in range(20)]
            for a, b in e:
                a.record(stream)
                fcall(stream)
                b.record(stream)
        stream.synchronize()
        flat = kstats([a.elapsed_time(b) for a, b in e], co_bytes)
        flat["copyout_over_flat"] = round(flat["avg_ms"] / kernels["ag_copyout"]["avg_ms"], 4)
        del fsrc, fdst, fplan, fcall

    # CU-budget sweep, after every full-GPU measurement (its small budgets
    # leave the GPU lightly loaded, and the next kernels would start while its
    # clocks come back up): each kernel confined to `budget` CUs by a CU-masked
    # stream (a hard budget), with one workgroup (4 waves, the default) and
    # four workgroups (16 waves) per CU; results are bit-identical by design
    sweep = []
    if not args.no_sweep:
        for budget in (8, 16, 32, 64, 128, 256):
            masked = tide.Stream(cus=range(budget))
            for wg in (1, 4):
                plan.set_options(**dict(opts, cu_budget=budget, wg_per_cu=wg))
                row = {"cu_budget": budget, "wg_per_cu": wg, "cu_masked": True}
                for name, call, nbytes in (("rs_local", rs_call, rs_bytes), ("ag_copyout", co_call, co_bytes)):
                    ms_ = masked.torch
                    call(ms_)
                    e = [(ev(), ev()) for _ in range(10)]
                    for a, b in e:
                        a.record(ms_)
                        call(ms_)
                        b.record(ms_)
                    ms_.synchronize()
                    avg = sum(a.elapsed_time(b) for a, b in e) / len(e)
                    row[name] = {"avg_ms": round(avg, 5), "gbps": round(nbytes / avg / 1e6, 1),
                                 "gbps_per_cu": round(nbytes / avg / 1e6 / budget, 2)}
                sweep.append(row)
            masked.destroy()
        plan.set_options(**opts)

    # CPU oracle on the same workload, streamed in groups of parameters, and a
    # bitwise check of this run's outputs against it
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_leg(w, plan, grads, outs, rank_major, params, rs_bytes + co_bytes, args.cpu_seconds)

    rs_k = kernels["rs_local"]
    achieved = rs_bytes / (rs_k["avg_ms"] * 1e-3) / 1e9
    # the committed counters are for the workload's own W and default options
    traffic = traffic_for(f"rs_local/{w.name}") if own_world else (None, None)
    value = (rs_bytes + co_bytes) / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "world": W, "params": w.nparams, "elements": sum_dk, "shard_elems": S,
                   "bytes_per_step": rs_bytes + co_bytes,
                   "options": {"rs_local": plan.options(0), "ag_copyout": plan.options(1)}},
        "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "rs_local_kernel", "unit_of_work": "one reduce-scatter call",
                     "launches_per_call": launches_per_call(plan, 0), "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic[0], "traffic_dram": traffic[1]},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "event_ms_per_step": round(step_ms_events, 5),
        "cu_sweep": sweep,
        "d2d_copy": d2d,
        "flat_copy": flat,
        "parity": parity,
        # elements per code path in the timed calls (vector, realigned, one by one)
        "paths": {"rs_local": plan.paths(0), "ag_copyout": plan.paths(1)},
        "stock_ab": stock_ab,
        "host_enqueue_us": host_us,
    }
    print(json.dumps(line), flush=True)
    if (parity and "MISMATCH" in parity.values()) or (stock_ab and stock_ab["shards"] != "bit-identical"):
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
