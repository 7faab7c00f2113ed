"""Randomized GPU parity over layouts and launch options.

Seeded random cases, each a random world size, a random list of parameter
shapes (empty tensors, fewer rows than ranks and 1-D tensors among them), a
random launch configuration (grid, workgroups per CU, chunk size, chunks per
wave per launch, LDS or global chunk table: so launches split inside and
between segments and rank-shard launch groups occur), misaligned gradient and
shard pointers, bf16 or fp32 gradients and a random Equation 5 epilogue; the
reduce-scatter, the copy-out and the copy-in must each match the oracle bit for
bit.
"""
import numpy as np
import pytest

from tests import gpu_util, oracle_pins
from tests.test_gpu_rs_variants import init_shards, random_shapes, run_rs

pytestmark = pytest.mark.gpu

CASES = 300


@pytest.fixture(scope="module")
def tide():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    return tide


def test_random_layouts_and_options(tide, oracle_mod):
    import torch

    seeds = np.random.default_rng(20261203).integers(1 << 30, size=CASES)
    for case, seed in enumerate(seeds):
        rng = np.random.default_rng(int(seed))
        W = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 24]))
        shapes = random_shapes(rng, W, int(rng.integers(1, 25)), max_k=int(rng.choice([8, 64, 300])))
        opts = dict(cu_budget=int(rng.integers(1, 9)), wg_per_cu=int(rng.integers(1, 3)),
                    chunk_elems=int(rng.choice([8, 16, 64, 256, 1024])), wave_chunks=int(rng.choice([1, 2, 3, 5, 64])),
                    flags=int(rng.choice([0, 0, tide.FLAG_NO_LDS])))
        what = f"case {case} (seed {seed}, W={W}, P={len(shapes)}, {opts})"
        plan = tide.Plan(W, shapes, **opts)
        f32 = bool(rng.random() < 0.3)
        grads = [[(oracle_pins.rand_f32 if f32 else oracle_pins.rand_bf16)(rng, s) for s in shapes] for _ in range(W)]
        alpha = float(rng.choice([1.0, 0.5, -2.0]))
        acc = bool(rng.random() < 0.4)
        init = init_shards(rng, W, plan.shard_elems) if acc else None
        offs = [[int(rng.integers(0, 9)) for _ in shapes] for _ in range(W)]
        got = run_rs(tide, plan, grads, alpha, acc, init, out_offset=int(rng.integers(0, 5)), grad_offsets=offs)
        want = oracle_mod.rs_local_ex(W, shapes, grads, alpha, acc, init, nthreads=8)
        for r in range(W):
            gpu_util.assert_same_f32(got[r], want[r], f"{what}: reduce-scatter rank {r}")
        X = [rng.standard_normal(s).astype(np.float32) for s in shapes]
        sh = oracle_pins.shards_of(W, shapes, X)
        rm_bits = oracle_mod.copyin(W, shapes, sh)
        rm = gpu_util.to_device_bf16(rm_bits)
        params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        tide.allgather_copyout(plan, rm, params)
        shards = [[torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in row] for row in sh]
        rm2 = torch.empty_like(rm)
        tide.allgather_copyin(plan, shards, rm2)
        torch.cuda.synchronize()
        want_co = oracle_mod.copyout(W, shapes, rm_bits)
        for p in range(len(shapes)):
            assert np.array_equal(gpu_util.bf16_bits(params[p]).reshape(shapes[p]), want_co[p]), f"{what}: copy-out {p}"
        assert np.array_equal(gpu_util.bf16_bits(rm2), rm_bits), f"{what}: copy-in"
    print(f"\n[random layouts] {CASES} cases bit-exact", flush=True)
