"""tide_plan_paths on the GPU: the report of which code path a call's elements
took agrees with the layouts that decide it, and the outputs stay bit-exact
on every path.  Layouts: aligned tensors (all vector bodies), every rank's
gradients at one common 2-byte phase (realigned bodies, or element by element
when few elements are off phase), ranks at different phases (element by
element), and a copy-out source off its destination's phase (realigned)."""
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


def _grads(W, shapes, phases, rng):
    """bf16 gradients as views starting phases[u] elements into their own
    buffers (torch allocations are 256-byte aligned), with host copies."""
    import torch

    host = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    dev = []
    for u in range(W):
        row = []
        for p, s in enumerate(shapes):
            n = int(np.prod(s))
            buf = torch.empty(n + 16, dtype=torch.bfloat16, device="cuda")
            v = buf[phases[u]:phases[u] + n]
            v.copy_(gpu_util.to_device_bf16(host[u][p]).reshape(-1))
            row.append(v.view(s))
        dev.append(row)
    return host, dev


@pytest.mark.parametrize("case", ["aligned", "one_phase", "one_phase_few", "mixed_phases"])
def test_reduce_scatter_paths(tide, oracle_mod, case):
    import torch

    W = 8
    rng = np.random.default_rng(11)
    shapes = [(W * 64, 256), (W * 32, 128)]
    if case == "one_phase_few":
        shapes = [(W * 64, 256), (W * 2, 8)]  # the off-phase tensor holds well under 1/50 of the elements
    phases = {"aligned": [0] * W, "one_phase": [1] * W, "one_phase_few": [0] * W,
              "mixed_phases": [u % 3 for u in range(W)]}[case]
    plan = tide.Plan(W, shapes)
    host, grads = _grads(W, shapes, phases, rng)
    if case == "one_phase_few":  # only the small tensor off phase
        for u in range(W):
            buf = torch.empty(grads[u][1].numel() + 16, dtype=torch.bfloat16, device="cuda")
            v = buf[1:1 + grads[u][1].numel()]
            v.copy_(grads[u][1].reshape(-1))
            grads[u][1] = v.view(shapes[1])
    outs = [torch.full((plan.shard_elems,), float("nan"), device="cuda") for _ in range(W)]
    tide.reduce_scatter_local(plan, grads, outs)
    torch.cuda.synchronize()
    want = oracle_mod.rs_local(W, shapes, host)
    for r in range(W):
        gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"{case} rank {r}")
    p = plan.paths(0)
    total = W * plan.shard_elems
    assert p["vector"] + p["realigned"] + p["element"] == total
    small = plan.numel[1]  # the second tensor's real elements, over all ranks' shards
    if case == "aligned":
        assert p == {"vector": total, "realigned": 0, "element": 0, "realigning_instance": False}
    elif case == "one_phase":
        assert p["realigning_instance"] is True and p["vector"] == 0
        assert p["realigned"] > 0.99 * total
    elif case == "one_phase_few":
        assert p["realigning_instance"] is False
        assert p["element"] == small and p["realigned"] == 0
    else:
        assert p == {"vector": 0, "realigned": 0, "element": total, "realigning_instance": False}


@pytest.mark.parametrize("phase", [0, 3])
def test_copyout_paths(tide, oracle_mod, phase):
    import torch

    W = 4
    shapes = [(W * 100, 64), (W * 40, 33)]
    plan = tide.Plan(W, shapes)
    rng = np.random.default_rng(3)
    X = [oracle_pins.rand_bf16(rng, s) for s in shapes]
    rm_bits = oracle_mod.pack(W, shapes, X)
    buf = torch.empty(rm_bits.size + 16, dtype=torch.bfloat16, device="cuda")
    rm = buf[phase:phase + rm_bits.size]
    rm.copy_(gpu_util.to_device_bf16(rm_bits))
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tide.allgather_copyout(plan, rm, params)
    torch.cuda.synchronize()
    for p_, x in zip(params, X):
        assert np.array_equal(gpu_util.bf16_bits(p_).reshape(x.shape), x)
    p = plan.paths(1)
    total = sum(plan.numel)
    assert p["vector"] + p["realigned"] + p["element"] == total
    if phase == 0:
        # the first tensor's rows are whole groups; the second's (33 per row) leave heads and tails
        assert p["realigned"] == 0 and p["vector"] >= plan.numel[0]
    else:
        assert p["realigned"] >= plan.numel[0] - 8 * W and p["vector"] < total // 2
