"""The seeded input generators: bf16 rounding and reproducibility."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-40).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8,
                  1.0 + 2.0**-9, 1.0 + 3 * 2.0**-9], dtype=np.float32),
        # exact ties at every exponent
        (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
    ])
    mine = synth.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rounding_keeps_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    bits = synth.bf16_bits_from_f32(x)
    assert np.all((bits & 0x7F80) == 0x7F80) and np.all((bits & 0x007F) != 0)


def test_host_generator_is_reproducible_and_scaled():
    w = synth.workload("tiny")
    a = synth.grads_host(w)
    b = synth.grads_host(w)
    assert all(np.array_equal(x, y) for ra, rb in zip(a, b) for x, y in zip(ra, rb))
    assert [g.shape for g in a[0]] == w.shapes
    # ranks draw from different streams
    assert not np.array_equal(a[0][2], a[1][2])


def test_outlier_recipe_scales_about_one_percent():
    w = synth.workload("llama3.1-70b-layer")
    small = synth.Workload(w.index, "probe", 2, [(1000, 100)], ["x"], sigma=1e-3, outliers=True)
    g = synth.grads_host(small)
    v = (g[0][0].astype(np.uint32) << 16).view(np.float32)
    frac = np.mean(np.abs(v) > 0.02)  # > 20 sigma of the unscaled part
    assert 0.005 < frac < 0.015


def test_workload_sizes():
    sizes = {}
    for name in synth.workloads.WORKLOAD_ORDER:
        w = synth.workload(name)
        sizes[name] = (w.world, w.nparams, sum(w.numel(p) for p in range(w.nparams)))
    assert sizes == {
        "tiny": (4, 4, 351),
        "llama3.1-8b-layer": (8, 9, 218112000),
        "llama3.1-70b-layer": (8, 9, 855654400),
        "qwen3-30b-a3b-moe-layer": (8, 393, 623120640),
        "wan2.2-dit-block": (8, 24, 351378944),
    }
