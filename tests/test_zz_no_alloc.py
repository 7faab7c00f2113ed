"""The allocation-free reduce-scatter (tide_reduce_scatter_local_noalloc),
called through the C ABI: bit for bit the results of
tide_reduce_scatter_local on the same inputs, on consecutive calls whose
tables overwrite each other in the device's scratch array (the second call
smaller than the first), under graph capture, and with a plan too large for
the scratch array refused before any device work."""
import ctypes

import numpy as np
import pytest

from tests import gpu_util, oracle_pins


def _call_noalloc(tide, plan, grad_ptrs, out_ptrs, alpha=1.0, accumulate=0, stream=0):
    return tide.lib.tide_reduce_scatter_local_noalloc(
        plan.handle, tide._ptr_array(grad_ptrs), tide._ptr_array(out_ptrs), ctypes.c_float(alpha), int(accumulate),
        ctypes.c_void_p(int(stream) or None))


def test_oversized_tables_are_refused_before_device_work():
    """Host only: a plan whose tables exceed the scratch array is a range
    error (the pointers are never touched)."""
    from param_collectives_amd import tide

    W, P = 8, 1500  # 1500 * 8 segments of 92 bytes > 1 MiB
    plan = tide.Plan(W, [(W, 8)] * P)
    fake = [0x10000 + 64 * i for i in range(W * P)]
    outs = [0x900000 + 64 * r for r in range(W)]
    assert _call_noalloc(tide, plan, fake, outs) == -2
    assert "at most" in tide.lib.tide_last_error().decode()
    small = tide.Plan(W, [(W, 8)] * 1000)  # fits: argument errors still come first
    assert _call_noalloc(tide, small, fake[: W * 1000], outs, accumulate=2) == -1
    fake[3] = 0
    assert _call_noalloc(tide, small, fake[: W * 1000], outs) == -1


def _case(tide, W, shapes, seed):
    import torch

    rng = np.random.default_rng(seed)
    plan = tide.Plan(W, shapes)
    host = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    grads = [[gpu_util.to_device_bf16(host[u][p]).view(shapes[p]) for p in range(len(shapes))] for u in range(W)]
    ref = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(W)]
    got = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(W)]
    ptrs = [grads[u][p].data_ptr() for u in range(W) for p in range(len(shapes))]
    return plan, grads, ptrs, ref, got


@pytest.mark.gpu
def test_noalloc_matches_the_allocating_entry_point():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    # first call: many segments (padding, a 1-D tail, tables of ~50 KB, so
    # several put launches); second call: a smaller plan whose tables
    # overwrite the start of the first's in the scratch array
    big_shapes = [(8 * 37 + 5, 64), (3, 130), (1000,)] * 25 + [(8 * 700, 96)]
    small_shapes = [(4 * 9 + 1, 33), (5,)]
    calls = [(8, big_shapes, 1, 1.0, 0), (4, small_shapes, 2, 0.25, 1)]
    s = torch.cuda.Stream()
    results = []
    for W, shapes, seed, alpha, acc in calls:
        plan, grads, ptrs, ref, got = _case(tide, W, shapes, seed)
        if acc:  # accumulate onto the same old values on both sides
            for a, b in zip(ref, got):
                a.normal_()
                b.copy_(a)
        torch.cuda.synchronize()
        plan.reduce_scatter_local_raw(ptrs, [o.data_ptr() for o in ref], alpha, acc, s.cuda_stream)
        assert _call_noalloc(tide, plan, ptrs, [o.data_ptr() for o in got], alpha, acc, s.cuda_stream) == 0, \
            tide.lib.tide_last_error()
        results.append((W, ref, got))
    torch.cuda.synchronize()
    for i, (W, ref, got) in enumerate(results):
        for r in range(W):
            gpu_util.assert_same_f32(got[r].cpu().numpy(), ref[r].cpu().numpy(), f"call {i} rank {r}")


@pytest.mark.gpu
def test_noalloc_runs_under_graph_capture():
    """The call enqueues kernel launches only, so a plan's first call can be
    captured (once the device has seen one call); every replay (new gradients
    written eagerly between them) matches the allocating entry point."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    W, shapes = 8, [(8 * 50 + 3, 40), (9,), (8 * 4, 300)]
    plan, grads, ptrs, ref, got = _case(tide, W, shapes, 3)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # one eager call on the device (with another plan) looks up the scratch
    # array's address; the captured call is this plan's first
    warm, _, wptrs, _, wout = _case(tide, 2, [(5, 3)], 4)
    assert _call_noalloc(tide, warm, wptrs, [o.data_ptr() for o in wout], 1.0, 0, s.cuda_stream) == 0
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        assert _call_noalloc(tide, plan, ptrs, [o.data_ptr() for o in got], 1.0, 0, s.cuda_stream) == 0
    for replay in range(3):
        for row in grads:
            for t in row:
                t.normal_()
        for o in got:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        plan.reduce_scatter_local_raw(ptrs, [o.data_ptr() for o in ref], 1.0, 0, 0)
        torch.cuda.synchronize()
        for r in range(W):
            gpu_util.assert_same_f32(got[r].cpu().numpy(), ref[r].cpu().numpy(), f"replay {replay} rank {r}")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["llama3.1-70b-layer", "qwen3-30b-a3b-moe-layer"])
def test_noalloc_full_size_layers(name):
    """Full-size layers: the Llama-3.1-70B layer (13 launches per call) and the
    Qwen3 MoE layer (3,144 segments: about 289 KB of tables, written by 73 put
    launches) give the allocating entry point's shards, bit for bit."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import synth
    from param_collectives_amd import tide

    w = synth.workload(name)
    plan = tide.Plan(w.world, w.shapes)
    grads = synth.grads_device(w, "cuda")
    ptrs = [grads[u][p].data_ptr() for u in range(w.world) for p in range(w.nparams)]
    ref = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    got = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(w.world)]
    plan.reduce_scatter_local_raw(ptrs, [o.data_ptr() for o in ref], 1.0, 0, 0)
    assert _call_noalloc(tide, plan, ptrs, [o.data_ptr() for o in got]) == 0, tide.lib.tide_last_error()
    torch.cuda.synchronize()
    for r in range(w.world):
        assert torch.equal(got[r].view(torch.int32), ref[r].view(torch.int32)), f"{name} rank {r}"
