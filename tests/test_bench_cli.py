"""The benchmark's command-line contract, on the CPU: it measures one GPU
only, and it refuses to run (rather than falling back to anything) when no
GPU is visible."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, BENCH, "--gpus", str(n)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_no_gpu_no_figures():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = subprocess.run([sys.executable, BENCH, "--steps", "1", "--warmup", "0"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1
    assert "no GPU visible" in r.stderr
    assert r.stdout == ""


def test_default_workload_is_the_largest_layer():
    """The headline line is quoted on the largest single-GPU workload."""
    import bench
    import synth

    assert bench.parse_args([]).workload == "llama3.1-70b-layer"
    sizes = {n: sum(synth.workload(n).numel(p) for p in range(synth.workload(n).nparams)) * synth.workload(n).world
             for n in synth.WORKLOADS}
    assert max(sizes, key=sizes.get) == bench.DEFAULT_WORKLOAD


@pytest.mark.parametrize("name,world,group_bytes", [("tiny", 4, 10 ** 9), ("tiny", 4, 300), ("mixed", 3, 20_000)])
def test_cpu_leg_streams_groups(name, world, group_bytes, monkeypatch):
    """The streamed oracle leg, run on CPU tensors: every group of parameters
    reproduces its range of the whole-plan oracle's outputs (so the verdict is
    bit-exact), and a flipped bit in one output is caught."""
    import dataclasses

    import numpy as np
    import torch

    import bench
    import oracle
    import synth
    from param_collectives_amd import tide

    w = synth.workload("tiny")
    if name == "mixed":  # several groups, padding rows, a parameter with fewer rows than ranks
        shapes = [(64, 33), (7,), (300, 5), (2, 9), (1000, 3), (41,)]
        w = dataclasses.replace(w, shapes=shapes, names=[f"p{i}" for i in range(len(shapes))], world=world)
    monkeypatch.setattr(bench, "GROUP_BYTES", group_bytes)
    groups = bench.param_groups(w, group_bytes)
    assert [p for g in groups for p in g] == list(range(w.nparams))
    assert all(len(g) == 1 or sum(2 * w.world * w.numel(p) for p in g) <= group_bytes for g in groups)
    if group_bytes < 10 ** 9:
        assert len(groups) > 1
    plan = tide.Plan(w.world, w.shapes)
    host = synth.grads_host(w)
    want = oracle.rs_local(w.world, w.shapes, host)
    X = synth.params_host(w)
    rm_bits = oracle.pack(w.world, w.shapes, X)

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    grads = [[t16(g) for g in row] for row in host]
    outs = [torch.from_numpy(o.copy()) for o in want]
    params = [t16(x) for x in X]
    rm = t16(rm_bits)
    cpu, parity = bench.cpu_leg(w, plan, grads, outs, rm, params, 10 ** 12, 0.01)
    assert parity == {"rs_local": "bit-exact", "ag_copyout": "bit-exact"}
    assert cpu["kind"] == "oracle" and cpu["single_thread_matches"] is True and cpu["value"] > 0
    assert f"{len(groups)} groups" in cpu["sample"]

    outs[w.world - 1].view(torch.int32)[-1] ^= 1
    params[-1].view(torch.int16).view(-1)[0] ^= 1
    _, parity = bench.cpu_leg(w, plan, grads, outs, rm, params, 10 ** 12, 0.01)
    assert parity == {"rs_local": "MISMATCH", "ag_copyout": "MISMATCH"}
