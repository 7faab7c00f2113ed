"""Interference study on one MI355X: what the collective's local kernels cost
the compute they overlap.

After "The Endgame of FSDP Communication" (Wang et al.), Section 2.2 ("SM
Wave Quantization", Equation 4, Figure 3), Table 4 (victim slowdown beside a
reduce-scatter) and Table 5 (the SM-id probe).  One GPU can show the part of
that cost that happens on the GPU running the collective: its kernels hold
CUs (wave slots, registers, LDS) and HBM bandwidth while a model kernel runs
beside them on another stream.

    python -m param_collectives_amd.interference --workload llama3.1-8b-layer \
        --out DIR [--profiles profiles]

Aggressors (one call each, repeated back to back on their own stream):
  tide-rs/grid=G     the layout-aware reduce-scatter, grid-limited to G
                     workgroups (one per CU), chunk table staged in LDS;
  tide-rs/noLDS/...  the same with the table left in global memory;
  tide-rs/mask=B     the same kernel on a stream masked to B CUs;
  stock              W stock gradient packs, then the fp32 reduce-scatter of
                     the packed buffers;
  copy-out           the all-gather copy-out (what the pages' direct landing
                     removes from the all-gather).
Victims (on a second stream): the 256 MiB elementwise kernel (y = a*x + b),
a small-M GEMM (256 x 8192 x 8192, bf16) and a large GEMM (8192^3, bf16), both
torch.matmul (the vendor GEMM library).  Reported per pair: the victim's p50
latency alone and beside the aggressor (only launches that ran entirely
inside the aggressor's run count), the slowdown, the aggressor's own time
alone and beside the victim, and its CU-ms per call (CUs held x time), the
analog of the pages' SM-ms per call.

Per call (Table 4's own measure, --per-call): the victim runs back to back on
its stream, and one aggressor call is released in the middle of that sequence
(the aggressor's stream waits for an event recorded after a fixed number of
victim launches).  The penalty of the call is the victims' extra time against
the same sequence without it; dividing it by the aggressor call's duration
gives the slowdown of the victim work that overlapped the call.  Configurations
add a disjoint split (the aggressor masked to 16 CUs, the victim to the other
240) and report the victim's own cost of that split.

Probe (Table 5's analog): 256 probe workgroups, each claiming a CU's whole LDS
and holding it 200 us, launched repeatedly during an aggressor's run: a
workgroup that starts after the first of them leaves was displaced.  Reported:
the displaced count (mode) and the share of probe launches with any.
"""
import argparse
import json
import math
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

ELEMENTWISE_ELEMS = 64 * 2**20  # 256 MiB of fp32 in, 256 MiB out
GEMMS = {"gemm_256x8192x8192": (256, 8192, 8192), "gemm_8192x8192x8192": (8192, 8192, 8192)}


def _median(v):
    return statistics.median(v) if v else float("nan")


class Study:
    def __init__(self, workload):
        import torch

        import synth
        from param_collectives_amd import tide

        self.torch, self.tide = torch, tide
        self.info = tide.device_info()
        self.w = w = synth.workload(workload)
        self.W = W = w.world
        self.plan = tide.Plan(W, w.shapes)
        self.S = S = self.plan.shard_elems
        self.sum_dk = sum(w.numel(p) for p in range(w.nparams))
        self.rs_bytes = 2 * W * self.sum_dk + 4 * W * S
        self.grads = synth.grads_device(w, "cuda")
        self.outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
        self.stream_v = tide.Stream()
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- parts

    def aggressor(self, kind, budget=None, masked=False, no_lds=False):
        """(call(stream), stream object, CUs held) for one aggressor."""
        tide, torch = self.tide, self.torch
        W, S = self.W, self.S
        flags = tide.FLAG_NO_LDS if no_lds else 0
        cus = self.info["cu_count"]
        if kind == "tide":
            grid = budget or cus
            plan = tide.Plan(W, self.w.shapes, cu_budget=grid, wg_per_cu=1, flags=flags)
            call = tide.reduce_scatter_call(plan, self.grads, self.outs)
            held = min(grid, cus)
            fn = call
        elif kind == "copyout":
            import synth

            rm = synth.rank_major_device(self.w, W * S, "cuda")
            params = [torch.empty(sh, dtype=torch.bfloat16, device="cuda") for sh in self.w.shapes]
            fn = tide.allgather_copyout_call(self.plan, rm, params)
            held = cus
        else:
            pack_plan = tide.Plan(W, [(W, S)])
            packed = [torch.empty(W * S, dtype=torch.float32, device="cuda") for _ in range(W)]
            stock_outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
            packs = [tide.stock_chunk_cat_call(self.plan, self.grads[u], packed[u]) for u in range(W)]
            red = tide.reduce_scatter_call(pack_plan, [[t.view(W, S)] for t in packed], stock_outs)

            def fn(stream):
                for c in packs:
                    c(stream)
                red(stream)

            held = cus
        stream = tide.Stream(cus=range(budget)) if masked else tide.Stream()
        if masked:
            held = budget
        return fn, stream, held

    def victim(self, name):
        torch, tide = self.torch, self.tide
        if name == "elementwise":
            x = torch.randn(ELEMENTWISE_ELEMS, device="cuda")
            y = torch.empty_like(x)
            return lambda s: tide.victim_axpb(x, y, 1.5, 0.25, stream=s)
        m, k, n = GEMMS[name]
        a = torch.randn(m, k, device="cuda").to(torch.bfloat16)
        b = torch.randn(k, n, device="cuda").to(torch.bfloat16)
        c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)

        def run(s):
            with torch.cuda.stream(s):
                torch.matmul(a, b, out=c)

        return run

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def time_alone(self, fn, stream, reps=10):
        torch = self.torch
        fn(stream)
        e = [(self.ev(), self.ev()) for _ in range(reps)]
        for a, b in e:
            a.record(stream)
            fn(stream)
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in e]

    def beside(self, agg_fn, agg_stream, vic_fn, t_agg, t_vic, nvic=20):
        """Aggressor calls back to back on its stream, victims on the other;
        returns (victim ms inside the aggressor's run, aggressor ms per call)."""
        torch = self.torch
        vs = self.stream_v.torch
        # enough aggressor calls to cover the victims even when slowed 4x
        k = max(3, min(3000, math.ceil((nvic * t_vic * 4.0 + 5.0) / max(t_agg, 1e-3))))
        a0, a1 = self.ev(), self.ev()
        torch.cuda.synchronize()
        a0.record(agg_stream)
        for _ in range(k):
            agg_fn(agg_stream)
        a1.record(agg_stream)
        marks = [(self.ev(), self.ev()) for _ in range(nvic)]
        for s, e in marks:
            s.record(vs)
            vic_fn(vs)
            e.record(vs)
        torch.cuda.synchronize()
        end = a0.elapsed_time(a1)
        inside = [s.elapsed_time(e) for s, e in marks if a0.elapsed_time(s) >= 0 and a0.elapsed_time(e) <= end]
        return inside, end / k

    def displaced(self, agg_fn, agg_stream, t_agg, launches=12, hold_ns=200_000):
        """Probe launches during the aggressor's run: per launch, the number of
        probe workgroups that started after the first one left."""
        torch, tide = self.torch, self.tide
        cus, lds = self.info["cu_count"], self.info["max_lds_per_workgroup"]
        vs = self.stream_v.torch
        recs = [torch.zeros(cus * tide.PROBE_WORDS, dtype=torch.int32, device="cuda") for _ in range(launches)]
        per = hold_ns * 1e-6 * 2.5
        k = max(3, min(3000, math.ceil((launches * per * 3.0 + 5.0) / max(t_agg, 1e-3))))
        a0, a1 = self.ev(), self.ev()
        torch.cuda.synchronize()
        a0.record(agg_stream)
        for _ in range(k):
            agg_fn(agg_stream)
        a1.record(agg_stream)
        marks = []
        for r in recs:
            s, e = self.ev(), self.ev()
            s.record(vs)
            tide.probe(r, cus, lds, hold_ns, stream=vs)
            e.record(vs)
            marks.append((s, e))
        torch.cuda.synchronize()
        end = a0.elapsed_time(a1)
        counts = []
        for (s, e), r in zip(marks, recs):
            if a0.elapsed_time(s) < 0 or a0.elapsed_time(e) > end:
                continue
            d = tide.decode_probe(r.cpu().numpy())
            counts.append(int((d["entry"] >= d["exit"].min()).sum()))
        return counts

    def per_call(self, agg_fn, agg_stream, vic_fn, vic_stream, t_vic, t_agg, reps=5, before=10):
        """One aggressor call released after `before` victim launches of a
        back-to-back victim sequence; returns per repetition (victim ms of the
        sequence with the call, without it, the call's own ms, victim launches
        that ran while the call did)."""
        torch = self.torch
        n = before + max(20, math.ceil(6.0 * t_agg / max(t_vic, 1e-3))) + 10
        out = []
        for _ in range(reps):
            row = []
            for with_call in (False, True):
                torch.cuda.synchronize()
                marks = [(self.ev(), self.ev()) for _ in range(n)]
                go = torch.cuda.Event()
                c0, c1 = self.ev(), self.ev()
                for i, (a, b) in enumerate(marks):
                    a.record(vic_stream)
                    vic_fn(vic_stream)
                    b.record(vic_stream)
                    if i == before - 1:
                        go.record(vic_stream)
                if with_call:
                    agg_stream.wait_event(go)
                    c0.record(agg_stream)
                    agg_fn(agg_stream)
                    c1.record(agg_stream)
                torch.cuda.synchronize()
                total = sum(a.elapsed_time(b) for a, b in marks)
                if with_call:
                    call = c0.elapsed_time(c1)
                    start, end = marks[0][0].elapsed_time(c0), marks[0][0].elapsed_time(c1)
                    overlap = sum(1 for a, b in marks
                                  if marks[0][0].elapsed_time(b) > start and marks[0][0].elapsed_time(a) < end)
                    row += [total, call, overlap]
                else:
                    row.append(total)
            base, total, call, overlap = row
            out.append((total, base, call, overlap))
        return out

    def run_per_call(self, configs, victims):
        torch, tide = self.torch, self.tide
        cus = self.info["cu_count"]
        results = {"device": self.info, "workload": self.w.name, "rs_bytes": self.rs_bytes, "victims": {},
                   "aggressors": []}
        vic = {name: self.victim(name) for name in victims}
        full = self.stream_v.torch
        rest = tide.Stream(cus=range(16, cus))  # the victim's side of the disjoint split
        for name, fn in vic.items():
            t = _median(self.time_alone(fn, full))
            t_rest = _median(self.time_alone(fn, rest.torch))
            results["victims"][name] = {"alone_p50_ms": round(t, 5), "alone_on_240_cus_p50_ms": round(t_rest, 5)}
        for label, kw in configs:
            disjoint = kw.pop("disjoint", False)
            fn, stream, held = self.aggressor(**kw)
            kw["disjoint"] = disjoint
            t_agg = _median(self.time_alone(fn, stream.torch))
            row = {"aggressor": label, "cus_held": held, "alone_ms": round(t_agg, 5)}
            for name, vfn in vic.items():
                vs = rest.torch if disjoint else full
                t_vic = results["victims"][name]["alone_on_240_cus_p50_ms" if disjoint else "alone_p50_ms"]
                reps = self.per_call(fn, stream.torch, vfn, vs, t_vic, t_agg)
                pen = [t - b for t, b, _, _ in reps]
                call = [c for _, _, c, _ in reps]
                p = _median(pen)
                c = _median(call)
                row[name] = {"penalty_ms": round(p, 5), "call_ms_beside": round(c, 5),
                             "overlap_slowdown_pct": round(100.0 * p / c, 2) if c > 0 else None,
                             "victims_overlapped": int(_median([o for _, _, _, o in reps])),
                             "penalty_ms_min": round(min(pen), 5), "penalty_ms_max": round(max(pen), 5)}
                if disjoint:
                    # what the split itself costs the victim: 240 CUs instead of 256
                    row[name]["split_cost_pct"] = round(
                        100.0 * (t_vic / results["victims"][name]["alone_p50_ms"] - 1.0), 2)
            results["aggressors"].append(row)
            print(json.dumps(row), flush=True)
            stream.destroy()
            torch.cuda.synchronize()
        rest.destroy()
        return results

    # ---------------------------------------------------------------- study

    def run(self, configs, victims):
        torch = self.torch
        results = {"device": self.info, "workload": self.w.name, "rs_bytes": self.rs_bytes, "victims": {},
                   "aggressors": []}
        vic = {name: self.victim(name) for name in victims}
        for name, fn in vic.items():
            t = self.time_alone(fn, self.stream_v.torch)
            results["victims"][name] = {"alone_p50_ms": round(_median(t), 5)}
        for label, kw in configs:
            fn, stream, held = self.aggressor(**kw)
            t_agg = _median(self.time_alone(fn, stream.torch))
            row = {"aggressor": label, "cus_held": held, "alone_ms": round(t_agg, 5),
                   "cu_ms_per_call": round(held * t_agg, 3)}
            for name, vfn in vic.items():
                alone = results["victims"][name]["alone_p50_ms"]
                # three runs, samples pooled: which stream's work the dispatcher
                # places first varies from run to run
                inside, per_call = [], []
                for _ in range(3):
                    got, pc = self.beside(fn, stream.torch, vfn, t_agg, alone)
                    inside += got
                    per_call.append(pc)
                p50 = _median(inside)
                row[name] = {"p50_ms": round(p50, 5), "slowdown_pct": round(100.0 * (p50 / alone - 1.0), 2),
                             "p10_ms": round(sorted(inside)[len(inside) // 10], 5) if inside else None,
                             "p90_ms": round(sorted(inside)[(9 * len(inside)) // 10], 5) if inside else None,
                             "samples": len(inside), "aggressor_ms_beside": round(_median(per_call), 5)}
            counts = self.displaced(fn, stream.torch, t_agg)
            row["probe"] = {"windows": len(counts),
                            "displaced_mode": statistics.mode(counts) if counts else None,
                            "displaced_max": max(counts) if counts else None,
                            "windows_hit_pct": round(100.0 * sum(c > 0 for c in counts) / len(counts), 1)
                            if counts else None}
            results["aggressors"].append(row)
            print(json.dumps(row), flush=True)
            stream.destroy()
            torch.cuda.synchronize()
        return results


DEFAULT_CONFIGS = [
    ("tide-rs grid=256", dict(kind="tide")),
    ("tide-rs grid=64", dict(kind="tide", budget=64)),
    ("tide-rs grid=16", dict(kind="tide", budget=16)),
    ("tide-rs noLDS grid=256", dict(kind="tide", no_lds=True)),
    ("tide-rs noLDS grid=16", dict(kind="tide", budget=16, no_lds=True)),
    ("tide-rs mask=64", dict(kind="tide", budget=64, masked=True)),
    ("tide-rs mask=16", dict(kind="tide", budget=16, masked=True)),
    ("stock pack+reduce", dict(kind="stock")),
    ("tide copy-out", dict(kind="copyout")),
]


PER_CALL_CONFIGS = [
    ("tide-rs grid=256", dict(kind="tide")),
    ("tide-rs grid=64", dict(kind="tide", budget=64)),
    ("tide-rs grid=16", dict(kind="tide", budget=16)),
    ("tide-rs mask=16", dict(kind="tide", budget=16, masked=True)),
    ("tide-rs noLDS grid=16", dict(kind="tide", budget=16, no_lds=True)),
    ("tide-rs noLDS mask=16", dict(kind="tide", budget=16, masked=True, no_lds=True)),
    ("tide-rs disjoint 16|240", dict(kind="tide", budget=16, masked=True, no_lds=True, disjoint=True)),
    ("stock pack+reduce", dict(kind="stock")),
    ("tide copy-out", dict(kind="copyout")),
]


def per_call_text(res, command):
    lines = [f"# Interference per call: {res['workload']} on one MI355X", "",
             f"command: {command}", f"device: {res['device']}", "",
             "victim p50 latency alone: " + ", ".join(
                 f"{k} {v['alone_p50_ms']:.4f} ms (on 240 CUs {v['alone_on_240_cus_p50_ms']:.4f} ms)"
                 for k, v in res["victims"].items()), "",
             "one aggressor call released in a back-to-back victim sequence: the victims' extra time (penalty, "
             "median of 5), the call's duration beside them, and penalty / call duration (the slowdown of the "
             "victim work the call overlapped); the disjoint split runs the victims on 240 CUs, the call on the "
             "other 16"]
    vics = list(res["victims"])
    head = f"{'aggressor':<26} {'CUs':>4} {'alone ms':>9} " + " ".join(
        f"{v[:18] + ' pen ms':>26} {'call ms':>8} {'overlap %':>9}" for v in vics)
    lines.append(head)
    for r in res["aggressors"]:
        cells = []
        for v in vics:
            x = r[v]
            cells.append(f"{x['penalty_ms']:>26.4f} {x['call_ms_beside']:>8.4f} {x['overlap_slowdown_pct']!s:>9}")
        lines.append(f"{r['aggressor']:<26} {r['cus_held']:>4} {r['alone_ms']:>9.4f} " + " ".join(cells))
    return "\n".join(lines) + "\n"


def summary_text(res, command):
    lines = [f"# Interference study: {res['workload']} on one MI355X", "",
             f"command: {command}", f"device: {res['device']}", "",
             "victim p50 latency alone: " + ", ".join(f"{k} {v['alone_p50_ms']:.4f} ms"
                                                     for k, v in res["victims"].items()), ""]
    vics = list(res["victims"])
    head = f"{'aggressor':<24} {'CUs':>4} {'ms/call':>8} {'CU-ms':>7} " + " ".join(f"{v[:22]:>22}" for v in vics) + \
        f" {'probe displaced (mode/max, % windows)':>38}"
    lines += ["slowdown of each victim beside the aggressor (%), aggressor time alone, probe displacement", head]
    for r in res["aggressors"]:
        pr = r["probe"]
        lines.append(f"{r['aggressor']:<24} {r['cus_held']:>4} {r['alone_ms']:>8.4f} {r['cu_ms_per_call']:>7.2f} " +
                     " ".join(f"{r[v]['slowdown_pct']:>21.1f}%" for v in vics) +
                     f" {str(pr['displaced_mode']) + '/' + str(pr['displaced_max']):>28} {pr['windows_hit_pct']!s:>8}")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="llama3.1-8b-layer")
    ap.add_argument("--out", required=True, help="folder for the JSON result")
    ap.add_argument("--profiles", default=None, help="also write the text summary here")
    ap.add_argument("--victims", default="elementwise," + ",".join(GEMMS))
    ap.add_argument("--per-call", action="store_true", help="one aggressor call inside a victim sequence")
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    study = Study(args.workload)
    if args.per_call:
        victims = [v for v in args.victims.split(",") if v != "gemm_8192x8192x8192"]
        res = study.run_per_call(PER_CALL_CONFIGS, victims)
        os.makedirs(args.out, exist_ok=True)
        with open(os.path.join(args.out, f"interference_per_call_{args.workload}.json"), "w") as f:
            json.dump(res, f, indent=1)
        cmd = f"python -m param_collectives_amd.interference --per-call --workload {args.workload} --out <out>"
        text = per_call_text(res, cmd)
        print(text, flush=True)
        if args.profiles:
            os.makedirs(args.profiles, exist_ok=True)
            with open(os.path.join(args.profiles, f"interference_per_call_{args.workload}.txt"), "w") as f:
                f.write(text)
        return
    res = study.run(DEFAULT_CONFIGS, args.victims.split(","))
    os.makedirs(args.out, exist_ok=True)
    with open(os.path.join(args.out, f"interference_{args.workload}.json"), "w") as f:
        json.dump(res, f, indent=1)
    cmd = f"python -m param_collectives_amd.interference --workload {args.workload} --out <out>"
    text = summary_text(res, cmd)
    print(text, flush=True)
    if args.profiles:
        os.makedirs(args.profiles, exist_ok=True)
        with open(os.path.join(args.profiles, f"interference_{args.workload}.txt"), "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
