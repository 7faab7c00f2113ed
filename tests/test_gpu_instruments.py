"""GPU checks of the interference instruments.

  * the elementwise victim against the oracle, bit for bit;
  * the hardware-ID probe against what the hardware itself enforces: with
    every probe workgroup claiming more than half of a CU's LDS, no two probe
    workgroups can share a CU at the same time, so records whose time
    intervals overlap must name different CUs, and no more CUs can appear
    than the device has (this pins the decoding of the ID registers);
  * a CU-masked stream confines the probe to the masked CUs;
  * the reduce-scatter on a CU-masked stream, and beside a running victim,
    still gives the oracle's shards.
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


@pytest.fixture(scope="module")
def info(tide):
    d = tide.device_info()
    print(f"\n[device] {d}", flush=True)
    return d


def ids(d):
    return d["xcc"] * 4096 + d["se"] * 512 + d["sh"] * 256 + d["cu"]


def max_concurrency_per_cu(d):
    """Largest number of records of one CU whose [entry, exit) intervals
    overlap at one moment."""
    worst = 0
    cu = ids(d)
    for c in np.unique(cu):
        m = cu == c
        ev = sorted([(t, 1) for t in d["entry"][m]] + [(t, -1) for t in d["exit"][m]], key=lambda e: (e[0], e[1]))
        cur = 0
        for _, step in ev:
            cur += step
            worst = max(worst, cur)
    return worst


def run_probe(tide, grid, lds, hold_ns, stream=None):
    import torch

    rec = torch.full((grid * tide.PROBE_WORDS,), -1, dtype=torch.int32, device="cuda")
    tide.probe(rec, grid, lds, hold_ns, stream=stream)
    torch.cuda.synchronize()
    return tide.decode_probe(rec.cpu().numpy())


@pytest.mark.parametrize("n,offset", [(0, 0), (1, 0), (7, 0), (4096 + 3, 0), (1 << 20, 0), (1 << 20, 1)])
def test_victim_matches_oracle(tide, oracle_mod, n, offset):
    import torch

    rng = np.random.default_rng(n + offset)
    x = rng.standard_normal(n).astype(np.float32)
    if n > 16:
        x[::97] = np.array([0x7FC00000, 0xFF800000, 0x00000001, 0x80000000, 0x7F7FFFFF], dtype=np.uint32).view(
            np.float32)[np.arange(len(x[::97])) % 5]
    for a, b in ((1.5, -0.25), (np.float32(1.0 + 2**-12), -1.0), (2.0, -3.0e38)):
        base = torch.from_numpy(np.concatenate([np.zeros(offset, np.float32), x])).cuda()
        out = torch.full((offset + n,), float("nan"), dtype=torch.float32, device="cuda")
        tide.victim_axpb(base[offset:], out[offset:], a, b)
        torch.cuda.synchronize()
        gpu_util.assert_same_f32(out[offset:].cpu().numpy(), oracle_mod.axpb(x, a, b), f"n={n} a={a} b={b}")


def test_probe_alone_one_workgroup_per_cu(tide, info):
    cus, lds = info["cu_count"], info["max_lds_per_workgroup"]
    if 2 * lds <= info["lds_per_cu"]:
        pytest.skip("a workgroup cannot claim more than half of a CU's LDS here")
    d = run_probe(tide, 2 * cus, lds, 100_000)
    assert np.array_equal(np.sort(d["block"]), np.arange(2 * cus))
    assert d["ok"].all()
    assert np.all(d["exit"] >= d["entry"])
    assert np.all(d["xcc"] < 8)
    assert max_concurrency_per_cu(d) == 1, "two probe workgroups on one CU at once: register decoding is wrong"
    distinct = len(np.unique(ids(d)))
    assert distinct <= cus
    first = d["block"] < cus
    on_xcc = np.bincount(d["xcc"][first], minlength=8)
    rr = float(np.mean(d["xcc"][first] == d["block"][first] % 8))
    print(f"[probe] distinct CUs {distinct} of {cus}; first {cus} workgroups per XCC {on_xcc.tolist()}; "
          f"workgroup b on XCC b mod 8 for {rr:.3f} of them", flush=True)


def test_probe_confined_by_cu_mask(tide, info):
    cus, lds = info["cu_count"], info["max_lds_per_workgroup"]
    if 2 * lds <= info["lds_per_cu"]:
        pytest.skip("a workgroup cannot claim more than half of a CU's LDS here")
    s = tide.Stream(cus=range(0, 32))
    try:
        d = run_probe(tide, 64, lds, 50_000, stream=s.torch)
    finally:
        s.destroy()
    distinct = len(np.unique(ids(d)))
    assert distinct <= 32
    assert max_concurrency_per_cu(d) == 1
    # 64 workgroups on at most 32 CUs: at least 32 had to wait for a first one to leave
    waited = int(np.sum(d["entry"] >= d["exit"].min()))
    assert waited >= 32, waited
    print(f"[probe] masked to 32 CUs: {distinct} distinct CUs, {waited} workgroups started in a second wave, "
          f"XCCs {sorted(set(d['xcc'].tolist()))}", flush=True)


def test_rs_on_masked_stream_and_beside_victim(tide, oracle_mod, info):
    import torch

    rng = np.random.default_rng(31)
    W = 8
    shapes = [(W * 300 + 5, 512), (1000,), (W * 64, 1024)]
    grads_h = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    want = oracle_mod.rs_local(W, shapes, grads_h, nthreads=8)
    plan = tide.Plan(W, shapes, cu_budget=16)
    grads = [[gpu_util.to_device_bf16(g).view(s) for g, s in zip(row, shapes)] for row in grads_h]
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
    x = torch.randn(1 << 24, device="cuda")
    y = torch.empty_like(x)
    masked = tide.Stream(cus=range(0, 16))
    other = tide.Stream()
    try:
        call = tide.reduce_scatter_call(plan, grads, outs)
        for _ in range(3):
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            call(masked.torch)
            tide.victim_axpb(x, y, 2.0, 1.0, stream=other.torch)
            torch.cuda.synchronize()
            for r in range(W):
                gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"rank {r}")
        gpu_util.assert_same_f32(y.cpu().numpy(), oracle_mod.axpb(x.cpu().numpy(), 2.0, 1.0), "victim")
    finally:
        masked.destroy()
        other.destroy()
