"""The benchmark's one JSON line, on the GPU: a short run of the default
workload (the Llama-3.1-70B layer) with the CPU-oracle leg, checked for every
field the report is read by, for internal consistency (rates against bytes
and times, the roofline fraction against its peak), and for the bitwise
parity verdict the run itself takes against the oracle."""
import json

import pytest

pytestmark = pytest.mark.gpu


def test_bench_line(capsys):
    import bench

    rc = bench.main(["--steps", "3", "--warmup", "1", "--no-sweep", "--no-extras", "--cpu-seconds", "1"])
    out = capsys.readouterr().out.strip().splitlines()
    assert rc == 0
    assert len(out) == 1, out
    d = json.loads(out[0])

    assert d["metric"] == bench.METRIC
    assert d["unit"] == "GB/s" and d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"] == "synthetic"
    cfg = d["config"]
    assert cfg["workload"] == "llama3.1-70b-layer" and cfg["world"] == 8 and cfg["params"] == 9
    assert cfg["elements"] == 855654400 and cfg["shard_elems"] == 106956800

    # the step's algorithmic bytes: reduce-scatter 2*W*sum(D*K) + 4*W*S, copy-out 4*sum(D*K)
    rs_bytes = 2 * 8 * cfg["elements"] + 4 * 8 * cfg["shard_elems"]
    co_bytes = 4 * cfg["elements"]
    assert cfg["bytes_per_step"] == rs_bytes + co_bytes
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(cfg["bytes_per_step"] / d["ms_per_step"] / 1e6, rel=1e-3)

    k = d["kernels"]
    assert k["rs_local"]["bytes"] == rs_bytes and k["ag_copyout"]["bytes"] == co_bytes
    for name in ("rs_local", "ag_copyout", "ag_copyin_f32"):
        assert k[name]["min_ms"] <= k[name]["median_ms"] <= k[name]["p90_ms"]
        assert k[name]["gbps"] == pytest.approx(k[name]["bytes"] / k[name]["avg_ms"] / 1e6, rel=1e-3)

    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["kernel"] == "rs_local_kernel" and r["launches_per_call"] >= 1
    assert r["achieved"] == pytest.approx(k["rs_local"]["gbps"], rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert 0 < r["frac"] < 1
    for key in ("traffic", "traffic_dram"):  # counters committed for this kernel source
        if r[key] is not None:
            assert r[key] == pytest.approx(rs_bytes, rel=0.05)

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GB/s" and c["value"] > 0 and c["cores"] >= 1
    assert c["single_thread_matches"] is True and c["sample"]
    assert d["parity"] == {"rs_local": "bit-exact", "ag_copyout": "bit-exact"}
    # the layer's tensors are aligned: every element of both timed operations takes a vector body
    assert d["paths"]["rs_local"] == {"vector": 8 * cfg["shard_elems"], "realigned": 0, "element": 0,
                                      "realigning_instance": False}
    assert d["paths"]["ag_copyout"]["vector"] == cfg["elements"]
