"""HIP graph capture of registered calls.

After one call with the same pointers (which uploads the plan's tables), a
call enqueues only kernel launches, so a step of calls can be captured once
and replayed.  Each replay here follows eager changes to the inputs (new
gradient values written in place, the outputs poisoned), and every replay's
outputs are checked bit for bit against the oracle on that replay's inputs.
"""
import numpy as np
import pytest

from tests import gpu_util, oracle_pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    return tide


def test_captured_step_replays_match_the_oracle(tide, oracle_mod):
    import torch

    rng = np.random.default_rng(77)
    W = 8
    shapes = [(W * 90 + 3, 130), (5,), (W * 16, 256), (3, 7)]
    # several launches per call, so that a replay also runs a sequence of kernels
    plan = tide.Plan(W, shapes, chunk_elems=256, wave_chunks=2)
    grads = [[torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes] for _ in range(W)]
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
    rm = torch.empty(W * plan.shard_elems, dtype=torch.bfloat16, device="cuda")
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    rs = tide.reduce_scatter_call(plan, grads, outs, alpha=0.5, accumulate=False)
    co = tide.allgather_copyout_call(plan, rm, params)

    def fill(seed):
        r = np.random.default_rng(seed)
        host = [[oracle_pins.rand_bf16(r, s) for s in shapes] for _ in range(W)]
        for u in range(W):
            for p in range(len(shapes)):
                grads[u][p].copy_(gpu_util.to_device_bf16(host[u][p]).view(shapes[p]))
        rm_bits = r.integers(0, 0x10000, size=W * plan.shard_elems, dtype=np.uint16)
        rm.copy_(gpu_util.to_device_bf16(rm_bits))
        for o in outs:
            o.fill_(float("nan"))
        for t in params:
            t.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        return host, rm_bits

    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rs()
        co()  # warm-up: binds the plan and uploads its tables
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rs()
        co()
    for replay in range(4):
        host, rm_bits = fill(1000 + replay)
        graph.replay()
        torch.cuda.synchronize()
        want = oracle_mod.rs_local_ex(W, shapes, host, 0.5, False)
        for r in range(W):
            gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"replay {replay} rank {r}")
        want_co = oracle_mod.copyout(W, shapes, rm_bits)
        for p in range(len(shapes)):
            assert np.array_equal(gpu_util.bf16_bits(params[p]).reshape(shapes[p]), want_co[p]), (replay, p)


def test_captured_copyin_and_fp32_reduce_scatter_replays(tide, oracle_mod):
    """The copy-in of fp32 shards and the reduce-scatter of fp32 gradients,
    captured after a warm-up call and replayed with new inputs written
    eagerly between the replays: every replay matches the oracle."""
    import torch

    W = 4
    shapes = [(W * 70 + 1, 96), (9,), (W * 8, 300)]
    plan = tide.Plan(W, shapes, wave_chunks=2)
    P = len(shapes)
    shards = [[torch.empty(plan.n_real[r][p], dtype=torch.float32, device="cuda") for p in range(P)]
              for r in range(W)]
    rm = torch.empty(W * plan.shard_elems, dtype=torch.bfloat16, device="cuda")
    grads = [[torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes] for _ in range(W)]
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
    ci = tide.allgather_copyin_call(plan, shards, rm)
    rs = tide.reduce_scatter_call(plan, grads, outs)

    def fill(seed):
        r = np.random.default_rng(seed)
        X = [r.standard_normal(s).astype(np.float32) for s in shapes]
        host_shards = oracle_pins.shards_of(W, shapes, X)
        for a in range(W):
            for p in range(P):
                shards[a][p].copy_(torch.from_numpy(np.ascontiguousarray(host_shards[a][p]).reshape(-1)))
        g = [[oracle_pins.rand_f32(r, s) for s in shapes] for _ in range(W)]
        for u in range(W):
            for p in range(P):
                grads[u][p].copy_(torch.from_numpy(g[u][p]))
        rm.view(torch.int16).fill_(-1)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        return host_shards, g

    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ci()
        rs()  # warm-up: binds the plan and uploads its tables
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ci()
        rs()
    for replay in range(3):
        host_shards, g = fill(500 + replay)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gpu_util.bf16_bits(rm), oracle_mod.copyin(W, shapes, host_shards)), replay
        want = oracle_mod.rs_local_ex(W, shapes, g)
        for r in range(W):
            gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"replay {replay} rank {r}")


def test_capture_refuses_set_up_and_uploads(tide, oracle_mod):
    """A call that would set up or upload the plan's tables while its stream
    is capturing is refused before it enqueues anything (first call, other
    pointers, other options); after a warm-up call with the same pointers the
    capture succeeds and its replays match the eager result."""
    import torch

    W = 4
    shapes = [(W * 33 + 2, 40), (7,)]
    plan = tide.Plan(W, shapes)
    rng = np.random.default_rng(5)
    host = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    grads = [[gpu_util.to_device_bf16(host[u][p]).view(shapes[p]) for p in range(len(shapes))] for u in range(W)]
    outs = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(W)]
    other = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(W)]
    rs = tide.reduce_scatter_call(plan, grads, outs)
    rs_other = tide.reduce_scatter_call(plan, grads, other)
    marker = torch.zeros(16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()

    def refused(call):
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(tide.TideError, match="capturing") as e:
            with torch.cuda.graph(graph, stream=s):
                marker.add_(1.0)  # the graph is never empty
                call()
        assert e.value.status == -1
        torch.cuda.synchronize()

    refused(lambda: rs(s))  # first call: the plan is not set up yet
    with torch.cuda.stream(s):
        rs()  # eager warm-up: set-up and uploads happen here
    torch.cuda.synchronize()
    want = oracle_mod.rs_local(W, shapes, host)
    for r in range(W):
        gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"eager rank {r}")
    refused(lambda: rs_other(s))  # other pointers: the call table would be re-uploaded
    for o in other:
        assert torch.isnan(o).all()  # nothing was enqueued for them

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rs()
    for replay in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for r in range(W):
            gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"replay {replay} rank {r}")

    plan.set_options(chunk_elems=512)  # new chunk table: must be uploaded eagerly first
    refused(lambda: rs(s))
    with torch.cuda.stream(s):
        rs()
    torch.cuda.synchronize()
    for r in range(W):
        gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"after new options, rank {r}")
