"""GPU parity of the reduce-scatter's Equation 5 terms and of the stock path.

Against the CPU oracle, bit for bit (any NaN matches any NaN):
  * alpha and accumulate on bf16 gradients (Equation 5), with special values
    in the accumulated shards;
  * fp32 gradients (the fp32 reduce-scatter of Section 4.3);
  * the stock gradient pack of one rank (Section 2.1, Equation 3);
and, as a property that holds at any size, the stock path (W packs, then the
fp32 reduce-scatter of the packed buffers) gives exactly the layout-aware
reduce-scatter's shards, at full layer size in the configuration the
benchmark times.
"""
import os

import numpy as np
import pytest

import synth
from tests import gpu_util, oracle_pins

pytestmark = pytest.mark.gpu

F32_SPECIALS = np.array([0x7FC00000, 0xFFC00001, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001,
                         0x80000001, 0x007FFFFF, 0x80000000, 0x00000000, 0x3F800000, 0x33800000],
                        dtype=np.uint32).view(np.float32)


@pytest.fixture(scope="module")
def tide():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    return tide


def upload(a, off=0):
    """numpy uint16 (bf16 bits) or float32 array -> device tensor placed
    `off` elements into a larger allocation (a misaligned pointer); returns
    (view, base)."""
    import torch

    flat = np.asarray(a).reshape(-1)
    if flat.dtype == np.uint16:
        base = gpu_util.to_device_bf16(np.concatenate([np.full(off, 0x7FC1, np.uint16), flat]))
    else:
        base = torch.from_numpy(np.concatenate([np.full(off, np.nan, np.float32), flat.astype(np.float32)])).cuda()
    return base[off:off + flat.size], base


def run_rs(tide, plan, grads, alpha=1.0, accumulate=False, init=None, out_offset=0, grad_offsets=None,
           guard=64):
    """The reduce-scatter on uploaded grads ([u][p] uint16 or float32 numpy);
    outputs start as `init` (W float32 arrays) or canaries; guard bands
    around every output must stay untouched.  Returns W float32 arrays."""
    import torch

    W, P = plan.world, len(plan.shapes)
    keep, dev = [], []
    for u in range(W):
        row = []
        for p in range(P):
            v, b = upload(grads[u][p], 0 if grad_offsets is None else grad_offsets[u][p])
            keep.append(b)
            row.append(v.view(plan.shapes[p]))
        dev.append(row)
    S = plan.shard_elems
    bases = []
    for r in range(W):
        b = torch.empty(out_offset + S + 2 * guard, dtype=torch.float32, device="cuda")
        b.view(torch.int32).fill_(0x7FC0DEAD)
        if init is not None:
            b[out_offset + guard:out_offset + guard + S] = torch.from_numpy(np.asarray(init[r], np.float32)).cuda()
        bases.append(b)
    outs = [b[out_offset + guard:out_offset + guard + S] for b in bases]
    tide.reduce_scatter_local(plan, dev, outs, alpha=alpha, accumulate=accumulate)
    torch.cuda.synchronize()
    res = []
    for b in bases:
        h = b.cpu().numpy()
        assert np.all(h[:out_offset + guard].view(np.uint32) == 0x7FC0DEAD), "guard band overwritten"
        assert np.all(h[out_offset + guard + S:].view(np.uint32) == 0x7FC0DEAD), "guard band overwritten"
        res.append(h[out_offset + guard:out_offset + guard + S])
    return res


def random_shapes(rng, world, count, max_k=200):
    shapes = []
    for _ in range(count):
        D = int(rng.integers(0, 3 * world + 6))
        shapes.append((D,) if rng.random() < 0.3 else (D, int(rng.integers(0, max_k + 1))))
    return shapes


def init_shards(rng, W, S):
    """Old shard values for accumulation: normals with special values mixed in."""
    out = []
    for _ in range(W):
        a = rng.standard_normal(S).astype(np.float32)
        m = rng.random(S) < 0.05
        a[m] = rng.choice(F32_SPECIALS, size=int(m.sum()))
        out.append(a)
    return out


def check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed, **kw):
    rng = np.random.default_rng(seed)
    plan = tide.Plan(world, shapes, **{k: v for k, v in kw.items() if k in ("chunk_elems", "flags", "cu_budget")})
    init = init_shards(rng, world, plan.shard_elems) if accumulate else None
    got = run_rs(tide, plan, grads, alpha, accumulate, init,
                 **{k: v for k, v in kw.items() if k in ("out_offset", "grad_offsets")})
    want = oracle_mod.rs_local_ex(world, shapes, grads, alpha, accumulate, init, nthreads=8)
    for r in range(world):
        gpu_util.assert_same_f32(got[r], want[r], f"W={world} alpha={alpha} acc={accumulate} rank {r}")


EPILOGUES = [(1.0, False), (0.125, False), (-3.0, False), (1e-3, False), (1.0, True), (0.37, True), (-0.0, True)]


@pytest.mark.parametrize("world", [1, 3, 4, 8, 16])
@pytest.mark.parametrize("alpha,accumulate", EPILOGUES)
def test_rs_alpha_accumulate_bf16(tide, oracle_mod, world, alpha, accumulate):
    rng = np.random.default_rng(100 + world)
    shapes = random_shapes(rng, world, 5) + [(world * 40 + 3, 64)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
    check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed=world)


@pytest.mark.parametrize("world", [1, 2, 3, 4, 8, 9])
@pytest.mark.parametrize("alpha,accumulate", [(1.0, False), (0.125, False), (0.37, True)])
def test_rs_fp32_grads(tide, oracle_mod, world, alpha, accumulate):
    rng = np.random.default_rng(200 + world)
    shapes = random_shapes(rng, world, 5) + [(world * 40 + 3, 64)]
    grads = [[oracle_pins.rand_f32(rng, s) for s in shapes] for _ in range(world)]
    check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed=world + 50)


def test_rs_fp32_misaligned_and_special_values(tide, oracle_mod):
    """Every source at its own element offset (no common vector phase, then
    a common one), fp32 special values, several chunk sizes."""
    rng = np.random.default_rng(7)
    W = 8
    shapes = [(W * 50 + 3, 37), (W * 16, 64), (5,)]
    grads = [[rng.choice(F32_SPECIALS, size=s) if p == 0 else oracle_pins.rand_f32(rng, s)
              for p, s in enumerate(shapes)] for _ in range(W)]
    ragged = [[int(rng.integers(0, 4)) for _ in shapes] for _ in range(W)]
    common = [[1 for _ in shapes] for _ in range(W)]
    for offs, out_offset, chunk in [(ragged, 0, 1024), (common, 1, 64), (None, 3, 8)]:
        check(tide, oracle_mod, W, shapes, grads, 1.0, False, seed=1, grad_offsets=offs, out_offset=out_offset,
              chunk_elems=chunk)
        check(tide, oracle_mod, W, shapes, grads, 0.5, True, seed=2, grad_offsets=offs, out_offset=out_offset,
              chunk_elems=chunk)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("world", [1, 3, 4, 8, 12])
def test_rs_every_source_phase(tide, oracle_mod, world, f32):
    """All ranks' gradients at one common element offset 0..3 against shards
    at offset 0 or 2: every phase of the realigned sum body (shifts of 1..3
    elements, for the templated and the any-W instances), with and without
    Equation 5's epilogue, several chunks per segment and ragged tails."""
    rng = np.random.default_rng(300 + world + (50 if f32 else 0))
    shapes = [(world * 40 + 3, 37), (world * 16, 64), (5,)]
    rand = oracle_pins.rand_f32 if f32 else oracle_pins.rand_bf16
    grads = [[rand(rng, s) for s in shapes] for _ in range(world)]
    for off in range(4):
        offs = [[off] * len(shapes) for _ in range(world)]
        for out_offset in (0, 2):
            for alpha, accumulate in ((1.0, False), (0.37, True)):
                check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed=off, grad_offsets=offs,
                      out_offset=out_offset, chunk_elems=64 if off % 2 else 1024)


@pytest.mark.parametrize("world", [3, 6, 12])
def test_rs_few_off_phase_segments(tide, oracle_mod, world):
    """Small 1-D parameters at the end of a layer whose shards start off a
    group boundary for some ranks (too few elements for the realigning
    instance): the plain instances sum those chunks element by element."""
    rng = np.random.default_rng(400 + world)
    shapes = [(world * 512, 256), (world * 64, 64), (31,), (61,), (world * 5 + 2,)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
    for alpha, accumulate in ((1.0, False), (0.37, True)):
        check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed=world)
        check(tide, oracle_mod, world, shapes, grads, alpha, accumulate, seed=world, chunk_elems=8)


def test_rs_accumulate_twice_is_two_additions(tide, oracle_mod):
    """Accumulating twice equals the oracle applied twice (the shards are read
    back each time, not cached)."""
    import torch

    rng = np.random.default_rng(8)
    W = 4
    shapes = [(W * 30 + 1, 70), (3,)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    plan = tide.Plan(W, shapes)
    dev = [[gpu_util.to_device_bf16(g).view(s) for g, s in zip(row, shapes)] for row in grads]
    init = init_shards(rng, W, plan.shard_elems)
    outs = [torch.from_numpy(a.copy()).cuda() for a in init]
    call = tide.reduce_scatter_call(plan, dev, outs, alpha=0.25, accumulate=True)
    call()
    call()
    torch.cuda.synchronize()
    want = oracle_mod.rs_local_ex(W, shapes, grads, 0.25, True, init)
    want = oracle_mod.rs_local_ex(W, shapes, grads, 0.25, True, want)
    for r in range(W):
        gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"rank {r}")


# ------------------------------------------------------------ stock pack


def run_pack(tide, plan, grads_u, offsets=None, packed_offset=0, guard=64):
    import torch

    keep, dev = [], []
    for p, g in enumerate(grads_u):
        v, b = upload(g, 0 if offsets is None else offsets[p])
        keep.append(b)
        dev.append(v.view(plan.shapes[p]))
    n = plan.world * plan.shard_elems
    base = torch.empty(packed_offset + n + 2 * guard, dtype=torch.float32, device="cuda")
    base.view(torch.int32).fill_(0x7FC0DEAD)
    tide.stock_chunk_cat(plan, dev, base[packed_offset + guard:packed_offset + guard + n])
    torch.cuda.synchronize()
    h = base.cpu().numpy()
    assert np.all(h[:packed_offset + guard].view(np.uint32) == 0x7FC0DEAD), "guard band overwritten"
    assert np.all(h[packed_offset + guard + n:].view(np.uint32) == 0x7FC0DEAD), "guard band overwritten"
    return h[packed_offset + guard:packed_offset + guard + n]


@pytest.mark.parametrize("world", [1, 3, 4, 8])
def test_stock_pack_matches_oracle(tide, oracle_mod, world):
    rng = np.random.default_rng(300 + world)
    shapes = random_shapes(rng, world, 6) + [(world * 40 + 3, 64)]
    grads_u = [oracle_pins.rand_bf16(rng, s) for s in shapes]
    want = oracle_mod.chunk_cat(world, shapes, grads_u)
    plan = tide.Plan(world, shapes)
    gpu_util.assert_same_f32(run_pack(tide, plan, grads_u), want, f"W={world}")
    offs = [int(rng.integers(0, 4)) for _ in shapes]
    for packed_offset, chunk in [(1, 8), (2, 64), (3, 4096)]:
        plan.set_options(chunk_elems=chunk)
        gpu_util.assert_same_f32(run_pack(tide, plan, grads_u, offs, packed_offset), want, f"W={world} {chunk}")


def stock_path(tide, plan, grads, outs, packed, pack_plan):
    """Stock FSDP2's reduce-scatter on one GPU: each rank packs its gradients
    into its own W*S fp32 buffer; rank r's shard is then the rank-order sum of
    the W buffers' r-th blocks (the fp32 reduce-scatter of a (W, S) plan)."""
    for u in range(plan.world):
        tide.stock_chunk_cat(plan, grads[u], packed[u])
    tide.reduce_scatter_local(pack_plan, [[p.view(plan.world, plan.shard_elems)] for p in packed], outs)


def test_stock_path_equals_layout_aware_rs(tide, oracle_mod):
    import torch

    rng = np.random.default_rng(11)
    W = 8
    shapes = random_shapes(rng, W, 6) + [(W * 40 + 3, 64), (6, 128)]
    grads_h = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    plan = tide.Plan(W, shapes)
    S = plan.shard_elems
    pack_plan = tide.Plan(W, [(W, S)])
    grads = [[gpu_util.to_device_bf16(g).view(s) for g, s in zip(row, shapes)] for row in grads_h]
    packed = [torch.empty(W * S, dtype=torch.float32, device="cuda") for _ in range(W)]
    stock = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
    layout = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(W)]
    stock_path(tide, plan, grads, stock, packed, pack_plan)
    tide.reduce_scatter_local(plan, grads, layout)
    torch.cuda.synchronize()
    want = oracle_mod.rs_local(W, shapes, grads_h)
    for r in range(W):
        gpu_util.assert_same_f32(stock[r].cpu().numpy(), want[r], f"stock rank {r}")
        gpu_util.assert_same_f32(layout[r].cpu().numpy(), want[r], f"layout-aware rank {r}")


# ------------------------------------------------------------ full size


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama3.1-8b-layer", "qwen3-30b-a3b-moe-layer"])
def test_full_size_stock_path_equals_layout_aware_rs(tide, name):
    """At full layer size, in the launch configuration the benchmark times:
    the stock path's shards are bit-identical to the layout-aware
    reduce-scatter's (whose full-size parity with the oracle is tested
    elsewhere)."""
    import torch

    w = synth.workload(name)
    print(f"\n[full-size stock] {name}: W={w.world} P={w.nparams}", flush=True)
    plan = tide.Plan(w.world, w.shapes)
    S = plan.shard_elems
    pack_plan = tide.Plan(w.world, [(w.world, S)])
    grads = synth.grads_device(w, "cuda")
    packed = [torch.empty(w.world * S, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    stock = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    layout = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    stock_path(tide, plan, grads, stock, packed, pack_plan)
    tide.reduce_scatter_local(plan, grads, layout)
    torch.cuda.synchronize()
    for r in range(w.world):
        a, b = stock[r].view(torch.int32), layout[r].view(torch.int32)
        diff = int((a != b).sum())
        assert diff == 0, f"{name} rank {r}: {diff} elements differ"
    print(f"[full-size stock] {name}: stock path == layout-aware RS, bit for bit", flush=True)


@pytest.mark.timeout(600)
def test_full_size_alpha_accumulate_and_fp32(tide, oracle_mod):
    """Llama-3.1-8B layer at full size: alpha and accumulate on bf16
    gradients, and fp32 gradients, against the oracle on every element."""
    import torch

    w = synth.workload("llama3.1-8b-layer")
    threads = min(16, os.cpu_count() or 1)
    plan = tide.Plan(w.world, w.shapes)
    S = plan.shard_elems
    rng = np.random.default_rng(12)
    init = [rng.standard_normal(S, dtype=np.float32) for _ in range(w.world)]
    print("\n[full-size eq5] bf16, alpha 0.125, accumulate", flush=True)
    grads = synth.grads_device(w, "cuda")
    outs = [torch.from_numpy(a).cuda() for a in init]
    tide.reduce_scatter_local(plan, grads, outs, alpha=0.125, accumulate=True)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    del outs
    host = [[gpu_util.bf16_bits(g).reshape(s) for g, s in zip(row, w.shapes)] for row in grads]
    del grads
    torch.cuda.empty_cache()
    want = oracle_mod.rs_local_ex(w.world, w.shapes, host, 0.125, True, init, nthreads=threads)
    del host
    for r in range(w.world):
        gpu_util.assert_same_f32(got[r], want[r], f"bf16 eq5 rank {r}")
    del got, want
    print("[full-size eq5] fp32 gradients", flush=True)
    grads = synth.grads_device(w, "cuda", dtype=torch.float32)
    outs = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    tide.reduce_scatter_local(plan, grads, outs)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    del outs
    host = [[g.cpu().numpy().reshape(s) for g, s in zip(row, w.shapes)] for row in grads]
    del grads
    torch.cuda.empty_cache()
    want = oracle_mod.rs_local_ex(w.world, w.shapes, host, nthreads=threads)
    for r in range(w.world):
        gpu_util.assert_same_f32(got[r], want[r], f"fp32 rank {r}")
    print("[full-size eq5] bit-exact", flush=True)


# ------------------------------------------------------------ split launches


@pytest.mark.parametrize("wave_chunks", [1, 3])
@pytest.mark.parametrize("world", [3, 8, 16])
def test_many_launches_per_call(tide, oracle_mod, world, wave_chunks):
    """Operations split into many launches (a few chunks per wave per launch,
    small grids) give the oracle's results for every operation and both
    gradient types; launch boundaries fall inside segments and between them,
    and with three rounds per launch the last launch is shorter."""
    import torch

    rng = np.random.default_rng(400 + world)
    shapes = random_shapes(rng, world, 5) + [(world * 40 + 3, 64), (7,)]
    opts = dict(cu_budget=3, wg_per_cu=1, chunk_elems=64, wave_chunks=wave_chunks)
    plan = tide.Plan(world, shapes, **opts)
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
    init = init_shards(rng, world, plan.shard_elems)
    got = run_rs(tide, plan, grads, alpha=0.5, accumulate=True, init=init)
    want = oracle_mod.rs_local_ex(world, shapes, grads, 0.5, True, init)
    for r in range(world):
        gpu_util.assert_same_f32(got[r], want[r], f"bf16 rank {r}")
    # rank shards that start off the 12-wave round grid open launch groups of
    # their own, so some launches start off that grid
    for op in (0, 4):
        assert np.any(plan.launches(op)[:, 0] % 12 != 0)
    g32 = [[oracle_pins.rand_f32(rng, s) for s in shapes] for _ in range(world)]
    got = run_rs(tide, plan, g32)
    want = oracle_mod.rs_local_ex(world, shapes, g32)
    for r in range(world):
        gpu_util.assert_same_f32(got[r], want[r], f"fp32 rank {r}")
    # copy-out, copy-in and the stock pack through the same many-launch options
    X = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    rm_bits = oracle_mod.copyin(world, shapes, oracle_pins.shards_of(world, shapes, X))
    rm = gpu_util.to_device_bf16(rm_bits)
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tide.allgather_copyout(plan, rm, params)
    shards = [[torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in row]
              for row in oracle_pins.shards_of(world, shapes, X)]
    rm2 = torch.empty_like(rm)
    tide.allgather_copyin(plan, shards, rm2)
    torch.cuda.synchronize()
    want_co = oracle_mod.copyout(world, shapes, rm_bits)
    for p in range(len(shapes)):
        assert np.array_equal(gpu_util.bf16_bits(params[p]).reshape(shapes[p]), want_co[p]), p
    assert np.array_equal(gpu_util.bf16_bits(rm2), rm_bits)
    gpu_util.assert_same_f32(run_pack(tide, plan, grads[0]), oracle_mod.chunk_cat(world, shapes, grads[0]), "pack")


def test_eq5_worked_golden_on_gpu(tide, oracle_mod):
    """The hand-worked Equation 5 cases (two roundings, scaled padding) on the
    GPU, against the golden bits."""
    from tests import goldens

    g = goldens.read("eq5_worked.txt")
    for c in sorted({k.split(".")[0] for k in g}):
        shape = (int(g[c + ".shape"][0][0]),)
        grads = [None, None]
        for row in g[c + ".grad"]:
            grads[int(row[0])] = [goldens.hex16(row[1:])]
        alpha = float(np.array([int(g[c + ".alpha"][0][0], 16)], dtype=np.uint32).view(np.float32)[0])
        acc = bool(int(g[c + ".accumulate"][0][0]))
        fp = lambda row: np.array([int(v, 16) for v in row[1:]], dtype=np.uint32).view(np.float32)
        old = [None, None]
        want = [None, None]
        for row in g[c + ".old"]:
            old[int(row[0])] = fp(row)
        for row in g[c + ".out"]:
            want[int(row[0])] = fp(row)
        plan = tide.Plan(2, [shape])
        got = run_rs(tide, plan, grads, alpha, acc, old)
        for r in range(2):
            gpu_util.assert_same_f32(got[r], want[r], f"case {c} rank {r}")
