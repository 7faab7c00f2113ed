"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

The bar is bit-exactness for both operations: the copy-out moves 16-bit
words, and the reduce-scatter sums in a fixed order (ranks 0..W-1, fp32), so
every output bit is determined (a NaN must meet a NaN).  Cases cover the
small workload, random shapes (empty, ragged, D < W, K = 1), every world-size
code path, misaligned tensors (scalar heads and tails), special values,
guard bands, every launch knob, and the four full-size layer workloads in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import synth
from tests import gpu_util, goldens, oracle_pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tide():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from param_collectives_amd import tide

    return tide


def run_rs(tide, plan, grads_bits, out_offset=0, grad_offsets=None, guard=64):
    """Upload grads (uint16 [u][p]), run the reduce-scatter, return the W
    outputs as numpy float32.  out_offset / grad_offsets place the tensors
    at that many elements into larger allocations (misaligned pointers);
    guard bands around every output are checked to be untouched."""
    import torch

    W, P = plan.world, len(plan.shapes)
    keep = []
    grads = []
    for u in range(W):
        row = []
        for p in range(P):
            off = 0 if grad_offsets is None else grad_offsets[u][p]
            flat = np.asarray(grads_bits[u][p], dtype=np.uint16).reshape(-1)
            base = gpu_util.to_device_bf16(np.concatenate([np.full(off, 0x7FC1, np.uint16), flat]))
            keep.append(base)
            row.append(base[off:].view(plan.shapes[p]) if flat.size else base[off:off].view(plan.shapes[p]))
        grads.append(row)
    S = plan.shard_elems
    bases = [torch.full((out_offset + S + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
             for _ in range(W)]
    for b in bases:
        b.view(torch.int32).fill_(0x7FC0DEAD)
    outs = [b[out_offset + guard:out_offset + guard + S] for b in bases]
    tide.reduce_scatter_local(plan, grads, outs)
    torch.cuda.synchronize()
    res = []
    for b in bases:
        h = b.cpu().numpy()
        g1 = h[:out_offset + guard].view(np.uint32)
        g2 = h[out_offset + guard + S:].view(np.uint32)
        assert np.all(g1 == 0x7FC0DEAD) and np.all(g2 == 0x7FC0DEAD), "guard band overwritten"
        res.append(h[out_offset + guard:out_offset + guard + S])
    return res


def run_copyout(tide, plan, rank_major_bits, param_offsets=None, rm_offset=0, guard=64):
    import torch

    P = len(plan.shapes)
    rm_base = gpu_util.to_device_bf16(np.concatenate([np.full(rm_offset, 0x7FC1, np.uint16),
                                                      np.asarray(rank_major_bits, np.uint16).reshape(-1)]))
    rm = rm_base[rm_offset:]
    bases, params = [], []
    for p in range(P):
        off = 0 if param_offsets is None else param_offsets[p]
        n = plan.numel[p]
        b = torch.empty(off + n + 2 * guard, dtype=torch.bfloat16, device="cuda")
        b.view(torch.int16).fill_(-1)  # 0xFFFF canary
        bases.append((b, off))
        params.append(b[off + guard:off + guard + n].view(plan.shapes[p]))
    tide.allgather_copyout(plan, rm, params)
    torch.cuda.synchronize()
    out = []
    for (b, off), p in zip(bases, range(P)):
        h = gpu_util.bf16_bits(b)
        n = plan.numel[p]
        assert np.all(h[:off + guard] == 0xFFFF) and np.all(h[off + guard + n:] == 0xFFFF), "guard band overwritten"
        out.append(h[off + guard:off + guard + n].reshape(plan.shapes[p]))
    return out


def random_shapes(rng, world, count, max_k=300):
    """1-D and 2-D shapes with D in [0, 3W+5] (D < W, D = 0 and ragged last
    ranks included) and K in [0, max_k]."""
    shapes = []
    for _ in range(count):
        D = int(rng.integers(0, 3 * world + 6))
        shapes.append((D,) if rng.random() < 0.3 else (D, int(rng.integers(0, max_k + 1))))
    return shapes


def check_rs(tide, oracle_mod, world, shapes, grads, **kw):
    plan = tide.Plan(world, shapes, **{k: v for k, v in kw.items() if k in ("cu_budget", "wg_per_cu",
                                                                            "chunk_elems", "flags")})
    got = run_rs(tide, plan, grads, **{k: v for k, v in kw.items() if k in ("out_offset", "grad_offsets")})
    want = oracle_mod.rs_local(world, shapes, grads, nthreads=8)
    for r in range(world):
        gpu_util.assert_same_f32(got[r], want[r], f"W={world} rank {r}")
    return got


# ---------------------------------------------------------------- small


def test_rs_tiny_workload(tide, oracle_mod):
    w = synth.workload("tiny")
    check_rs(tide, oracle_mod, w.world, w.shapes, synth.grads_host(w))


def test_rs_worked_example(tide, oracle_mod):
    g = goldens.read("rs_worked.txt")
    W = int(g["world"][0][0])
    shapes = [tuple(goldens.ints(s)) for s in g["shape"]]
    grads = [[None] for _ in range(W)]
    for row in g["grad"]:
        grads[int(row[0])][0] = goldens.hex16(row[1:]).reshape(shapes[0])
    check_rs(tide, oracle_mod, W, shapes, grads)


def test_copyout_tiny_round_trip(tide, oracle_mod):
    w = synth.workload("tiny")
    X = synth.params_host(w)
    plan = tide.Plan(w.world, w.shapes)
    rm = oracle_mod.pack(w.world, w.shapes, X)
    geo = oracle_mod.plan(w.world, w.shapes)
    for p in range(w.nparams):  # padding slots hold canaries that must not be read
        for r in range(w.world):
            a = geo["rank_major_offset"][p, r]
            rm[a + geo["n_real"][p, r]:a + geo["n"][p]] = 0x7FC1
    back = run_copyout(tide, plan, rm)
    for p in range(w.nparams):
        assert np.array_equal(back[p], X[p])


@pytest.mark.parametrize("world", [1, 2, 3, 4, 5, 8, 16, 64])
def test_rs_random_shapes(tide, oracle_mod, world):
    rng = np.random.default_rng(100 + world)
    for trial in range(3):
        shapes = random_shapes(rng, world, int(rng.integers(1, 6)))
        shapes.append((world * 37 + 3, 129))  # several chunks and a ragged tail
        grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
        check_rs(tide, oracle_mod, world, shapes, grads, chunk_elems=512)


def test_rs_largest_world(tide, oracle_mod):
    """W = 256, the largest world a plan accepts: 256 sources per segment on
    the generic path, most ranks holding only padding."""
    rng = np.random.default_rng(123)
    world = 256
    shapes = [(300, 2), (1,), (513, 3), (256 * 3, 8)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
    check_rs(tide, oracle_mod, world, shapes, grads, chunk_elems=8)
    check_rs(tide, oracle_mod, world, shapes, grads)


@pytest.mark.parametrize("world", [1, 3, 4, 8])
def test_copyout_random_shapes(tide, oracle_mod, world):
    rng = np.random.default_rng(200 + world)
    for trial in range(3):
        shapes = random_shapes(rng, world, int(rng.integers(1, 6)))
        shapes.append((world * 41 + 5, 257))
        plan = tide.Plan(world, shapes, chunk_elems=512)
        rm = rng.integers(0, 0x10000, size=world * plan.shard_elems, dtype=np.uint16)
        got = run_copyout(tide, plan, rm)
        want = oracle_mod.copyout(world, shapes, rm)
        for p in range(len(shapes)):
            assert np.array_equal(got[p], want[p]), (world, shapes, p)


def test_rs_misaligned_tensors(tide, oracle_mod):
    """Tensors starting off a 16-byte boundary: the same phase on every rank
    (scalar head, vector body) and different phases (scalar path)."""
    rng = np.random.default_rng(7)
    W = 8
    shapes = [(W * 50 + 3, 77), (13,), (W * 9, 64)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    for same in (True, False):
        for out_offset in (0, 1, 2, 3):
            offs = [[(3 if same else (u + p) % 8) for p in range(len(shapes))] for u in range(W)]
            check_rs(tide, oracle_mod, W, shapes, grads, out_offset=out_offset, grad_offsets=offs, chunk_elems=256)


def test_copyout_misaligned_tensors(tide, oracle_mod):
    rng = np.random.default_rng(8)
    W = 4
    shapes = [(W * 70 + 1, 45), (9,), (W * 8, 64)]
    plan = tide.Plan(W, shapes, chunk_elems=256)
    rm = rng.integers(0, 0x10000, size=W * plan.shard_elems, dtype=np.uint16)
    want = oracle_mod.copyout(W, shapes, rm)
    for rm_offset in (0, 1, 5):
        for poffs in ([0, 0, 0], [1, 2, 3], [5, 5, 5], [7, 0, 4]):
            got = run_copyout(tide, plan, rm, param_offsets=poffs, rm_offset=rm_offset)
            for p in range(len(shapes)):
                assert np.array_equal(got[p], want[p]), (rm_offset, poffs, p)


def test_copies_every_source_phase(tide, oracle_mod):
    """Every 16-byte phase of the source against an aligned destination (and
    against a destination at phase 3): the copy-out's and the bf16 copy-in's
    realigned bodies for shifts of 1..7 elements, the fp32 copy-in's for 1..3,
    with ragged tails and several chunks per segment."""
    rng = np.random.default_rng(31)
    for W, shapes, chunk in ((1, [(4099,), (37, 29)], 256), (3, [(3 * 37 + 1, 29), (1001,)], 64)):
        plan = tide.Plan(W, shapes, chunk_elems=chunk)
        rm = rng.integers(0, 0x10000, size=W * plan.shard_elems, dtype=np.uint16)
        want = oracle_mod.copyout(W, shapes, rm)
        for rm_offset in range(8):
            for poff in (0, 3):
                got = run_copyout(tide, plan, rm, param_offsets=[poff] * len(shapes), rm_offset=rm_offset)
                for p in range(len(shapes)):
                    assert np.array_equal(got[p], want[p]), (W, rm_offset, poff, p)
        X = [rng.standard_normal(s).astype(np.float32) for s in shapes]
        shards = oracle_pins.shards_of(W, shapes, X)
        cwant = oracle_mod.copyin(W, shapes, shards)
        bits = [rng.integers(0, 0x10000, size=s, dtype=np.uint16) for s in shapes]
        bshards = oracle_pins.shards_of(W, shapes, bits)
        bwant = oracle_mod.copyin(W, shapes, bshards)
        for off in range(8):
            offs = [[off] * len(shapes) for _ in range(W)]
            assert np.array_equal(run_copyin(tide, plan, shards, shard_offsets=offs), cwant), (W, off, "fp32")
            assert np.array_equal(run_copyin(tide, plan, bshards, shard_offsets=offs), bwant), (W, off, "bf16")


def test_rs_special_values(tide, oracle_mod):
    rng = np.random.default_rng(9)
    W = 8
    shapes = [(W * 64, 33)]
    specials = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x8000, 0x0000, 0x0080,
                         0x3F80], dtype=np.uint16)
    grads = [[rng.choice(specials, size=s) for s in shapes] for _ in range(W)]
    check_rs(tide, oracle_mod, W, shapes, grads, chunk_elems=1024)


def test_knobs_do_not_change_results(tide, oracle_mod):
    """Section 4.3: CTA counts and chunk sizes leave every output bit as is."""
    rng = np.random.default_rng(10)
    W = 8
    shapes = [(W * 100 + 5, 96), (6, 40), (1000,), (W * 3, 4096)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    want = oracle_mod.rs_local(W, shapes, grads, nthreads=8)
    rm = rng.integers(0, 0x10000, size=W * tide.Plan(W, shapes).shard_elems, dtype=np.uint16)
    want_co = oracle_mod.copyout(W, shapes, rm)
    knobs = [dict(), dict(cu_budget=1, wg_per_cu=1), dict(cu_budget=3, wg_per_cu=2, chunk_elems=8),
             dict(cu_budget=64, wg_per_cu=4, chunk_elems=65536), dict(flags=1), dict(flags=2), dict(flags=3),
             dict(cu_budget=256, wg_per_cu=16, chunk_elems=1024, flags=3), dict(flags=4),
             dict(cu_budget=7, wg_per_cu=3, chunk_elems=64, flags=7), dict(wave_chunks=1),
             dict(cu_budget=2, wg_per_cu=1, chunk_elems=8, wave_chunks=3),
             dict(cu_budget=5, wg_per_cu=2, chunk_elems=64, wave_chunks=2, flags=4)]
    for kw in knobs:
        plan = tide.Plan(W, shapes, **kw)
        got = run_rs(tide, plan, grads)
        for r in range(W):
            gpu_util.assert_same_f32(got[r], want[r], f"{kw} rank {r}")
        co = run_copyout(tide, plan, rm)
        for p in range(len(shapes)):
            assert np.array_equal(co[p], want_co[p]), (kw, p)


def test_repeat_calls_and_pointer_table_changes(tide, oracle_mod):
    """A plan reused with new tensors uploads its new pointer table; repeated
    calls give identical bits."""
    import torch

    rng = np.random.default_rng(11)
    W = 4
    shapes = [(W * 20 + 1, 50), (7,)]
    plan = tide.Plan(W, shapes, chunk_elems=128)
    for trial in range(3):
        grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
        want = oracle_mod.rs_local(W, shapes, grads)
        dev = [[gpu_util.to_device_bf16(g).view(s) for g, s in zip(row, shapes)] for row in grads]
        outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
        for _ in range(2):
            tide.reduce_scatter_local(plan, dev, outs)
            torch.cuda.synchronize()
            for r in range(W):
                gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"trial {trial} rank {r}")


def test_launch_table_slice_staged_or_not(tide, oracle_mod):
    """Each launch stages its own slice of the chunk-to-segment table in LDS
    when it fits.  Here the first copy-out launch covers 16,384 one-element
    segments, one more than fits, so it reads its slice from global memory,
    and the second covers the 8 segments of one large parameter (staged)."""
    W = 8
    shapes = [(8,)] * 2048 + [(8, 8 * 1024 * 1024)]
    # 1024 waves, 32 rounds of 4096-element chunks, 16 rounds per launch
    plan = tide.Plan(W, shapes, cu_budget=256, wg_per_cu=1, wave_chunks=16)
    assert len(plan.segments(1)) == 2048 * W + W
    assert plan.options(1)["chunk_elems"] == 4096
    rng = np.random.default_rng(88)
    rm_bits = rng.integers(0, 0x10000, size=W * plan.shard_elems, dtype=np.uint16)
    got = run_copyout(tide, plan, rm_bits)
    want = oracle_mod.copyout(W, shapes, rm_bits)
    for p in range(len(shapes)):
        assert np.array_equal(got[p], want[p]), p


def test_empty_work_is_a_no_op(tide):
    import torch

    plan = tide.Plan(4, [(0, 8), (3, 0)])
    assert plan.shard_elems == 0
    grads = [[torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in plan.shapes] for _ in range(4)]
    outs = [torch.empty(0, dtype=torch.float32, device="cuda") for _ in range(4)]
    tide.reduce_scatter_local(plan, grads, outs)
    tide.allgather_copyout(plan, torch.empty(0, dtype=torch.bfloat16, device="cuda"),
                           [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in plan.shapes])
    torch.cuda.synchronize()


def test_streams_are_honoured(tide, oracle_mod):
    import torch

    rng = np.random.default_rng(12)
    W = 8
    shapes = [(W * 64, 512)]
    grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    want = oracle_mod.rs_local(W, shapes, grads)
    plan = tide.Plan(W, shapes)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev = [[gpu_util.to_device_bf16(g).view(sh) for g, sh in zip(row, shapes)] for row in grads]
        outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
        tide.reduce_scatter_local(plan, dev, outs)
    s.synchronize()
    for r in range(W):
        gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"rank {r}")


# ------------------------------------------------------------ full size

# the four layers, and the smaller context shape class (16 equal tensors, 32 MiB of fp32 shard per rank)
FULL = ["llama3.1-8b-layer", "llama3.1-70b-layer", "qwen3-30b-a3b-moe-layer", "wan2.2-dit-block", "equal16-32mib"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_bit_exact(tide, oracle_mod, name):
    """Every output element of both operations at the full layer shapes,
    with the launch options the benchmark times (the library defaults)."""
    import os

    import torch

    w = synth.workload(name)
    print(f"\n[full-size] {name}: W={w.world} P={w.nparams}", flush=True)
    plan = tide.Plan(w.world, w.shapes)
    grads = synth.grads_device(w, "cuda")
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(w.world)]
    tide.reduce_scatter_local(plan, grads, outs)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    del outs
    host = [[gpu_util.bf16_bits(g).reshape(s) for g, s in zip(row, w.shapes)] for row in grads]
    del grads
    torch.cuda.empty_cache()
    threads = min(16, os.cpu_count() or 1)
    want = oracle_mod.rs_local(w.world, w.shapes, host, nthreads=threads)
    del host
    for r in range(w.world):
        gpu_util.assert_same_f32(got[r], want[r], f"{name} rank {r}")
    print(f"[full-size] {name}: reduce-scatter bit-exact, max abs error 0", flush=True)
    del got, want
    # copy-out
    rm = synth.rank_major_device(w, w.world * plan.shard_elems, "cuda")
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in w.shapes]
    tide.allgather_copyout(plan, rm, params)
    torch.cuda.synchronize()
    want_co = oracle_mod.copyout(w.world, w.shapes, gpu_util.bf16_bits(rm), nthreads=threads)
    for p in range(w.nparams):
        assert np.array_equal(gpu_util.bf16_bits(params[p]).reshape(w.shapes[p]), want_co[p]), (name, p)
    print(f"[full-size] {name}: copy-out bit-exact", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("world,shape", [(1, (2**31 + 1000,)), (2, (2**31 + 3 * 1024 + 5,))])
def test_offsets_beyond_two_to_the_31(tide, oracle_mod, world, shape):
    """One tensor of more than 2^31 elements (byte offsets beyond 2^32, a
    segment longer than 2^31 elements when W = 1, a ragged last rank when
    W = 2): every output element of both operations."""
    import torch

    print(f"\n[int64] W={world} shape={shape}", flush=True)
    plan = tide.Plan(world, [shape])
    g = torch.Generator(device="cuda")
    g.manual_seed(31 + world)
    grads = [[torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)]
             for _ in range(world)]
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(world)]
    tide.reduce_scatter_local(plan, grads, outs)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    del outs
    host = [[gpu_util.bf16_bits(row[0]).reshape(shape)] for row in grads]
    want = oracle_mod.rs_local(world, [shape], host, nthreads=world)
    for r in range(world):
        gpu_util.assert_same_f32(got[r], want[r], f"rank {r}")
    del got, want
    # copy-out of the same size: the gradients of rank 0 padded into a rank-major buffer
    rm = torch.empty(world * plan.shard_elems, dtype=torch.bfloat16, device="cuda")
    rm.view(torch.int16).fill_(0x7FC1)
    flat = grads[0][0].reshape(-1)
    n = plan.shard_elems
    for r in range(world):
        lo, hi = r * n, min((r + 1) * n, flat.numel())
        if hi > lo:
            rm[r * n:r * n + (hi - lo)] = flat[lo:hi]
    param = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    tide.allgather_copyout(plan, rm, [param])
    torch.cuda.synchronize()
    assert torch.equal(param.view(torch.int16), grads[0][0].view(torch.int16))


# ------------------------------------------------------------ copy-in


def run_copyin(tide, plan, shard_bits_or_f32, shard_offsets=None, guard=64):
    """Upload shards ([r][p] numpy uint16 bf16 bits or float32), run the
    copy-in into a canary-filled rank-major buffer with guard bands, return
    the rank-major buffer as uint16."""
    import torch

    W, P = plan.world, len(plan.shapes)
    keep, shards = [], []
    for r in range(W):
        row = []
        for p in range(P):
            a = np.asarray(shard_bits_or_f32[r][p]).reshape(-1)
            off = 0 if shard_offsets is None else shard_offsets[r][p]
            if a.dtype == np.uint16:
                base = gpu_util.to_device_bf16(np.concatenate([np.full(off, 0x7FC1, np.uint16), a]))
            else:
                base = torch.from_numpy(np.concatenate([np.full(off, np.nan, np.float32), a])).cuda()
            keep.append(base)
            row.append(base[off:])
        shards.append(row)
    n = W * plan.shard_elems
    buf = torch.empty(n + 2 * guard, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(0x7FC1)
    tide.allgather_copyin(plan, shards, buf[guard:guard + n])
    torch.cuda.synchronize()
    h = gpu_util.bf16_bits(buf)
    assert np.all(h[:guard] == 0x7FC1) and np.all(h[guard + n:] == 0x7FC1), "guard band overwritten"
    return h[guard:guard + n]


@pytest.mark.parametrize("f32", [True, False], ids=["fp32", "bf16"])
def test_copyin_tiny_and_round_trip(tide, oracle_mod, f32):
    w = synth.workload("tiny")
    rng = np.random.default_rng(20)
    X = [rng.standard_normal(s).astype(np.float32) if f32 else rng.integers(0, 0x10000, size=s, dtype=np.uint16)
         for s in w.shapes]
    shards = oracle_pins.shards_of(w.world, w.shapes, X)
    plan = tide.Plan(w.world, w.shapes)
    got = run_copyin(tide, plan, shards)
    want = oracle_mod.copyin(w.world, w.shapes, shards)
    assert np.array_equal(got, want)
    # GPU round trip: copy-in then copy-out gives the (cast) parameters back
    back = run_copyout(tide, plan, got)
    for p in range(w.nparams):
        ref = oracle_mod.cast_bf16(X[p]).reshape(w.shapes[p]) if f32 else X[p]
        assert np.array_equal(back[p], ref)


@pytest.mark.parametrize("world", [1, 3, 4, 8])
@pytest.mark.parametrize("f32", [True, False], ids=["fp32", "bf16"])
def test_copyin_random_shapes(tide, oracle_mod, world, f32):
    rng = np.random.default_rng(300 + world + 7 * f32)
    for trial in range(3):
        shapes = random_shapes(rng, world, int(rng.integers(1, 6)))
        shapes.append((world * 43 + 5, 257))
        X = [(rng.standard_normal(s) * 10).astype(np.float32) if f32 else
             rng.integers(0, 0x10000, size=s, dtype=np.uint16) for s in shapes]
        shards = oracle_pins.shards_of(world, shapes, X)
        plan = tide.Plan(world, shapes, chunk_elems=512)
        assert np.array_equal(run_copyin(tide, plan, shards), oracle_mod.copyin(world, shapes, shards)), shapes


def test_copyin_misaligned_and_special_values(tide, oracle_mod):
    rng = np.random.default_rng(21)
    W = 4
    shapes = [(W * 60 + 3, 37), (11,), (W * 8, 64)]
    specials = np.array([0x7FC00001, 0x7F800001, 0xFFA10000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x3F808000,
                         0x3F818000, 0x00008000, 0x00018000, 0x80000000, 0x007FFFFF], dtype=np.uint32).view(np.float32)
    X = [np.where(rng.random(s) < 0.2, rng.choice(specials, size=s), rng.standard_normal(s)).astype(np.float32)
         for s in shapes]
    shards = oracle_pins.shards_of(W, shapes, X)
    want = oracle_mod.copyin(W, shapes, shards)
    plan = tide.Plan(W, shapes, chunk_elems=256)
    for offs in ([[0] * 3] * W, [[1, 2, 3]] * W, [[(r + p) % 4 for p in range(3)] for r in range(W)]):
        assert np.array_equal(run_copyin(tide, plan, shards, shard_offsets=offs), want), offs
    bits = [rng.integers(0, 0x10000, size=s, dtype=np.uint16) for s in shapes]
    bshards = oracle_pins.shards_of(W, shapes, bits)
    bwant = oracle_mod.copyin(W, shapes, bshards)
    for offs in ([[0] * 3] * W, [[1, 3, 5]] * W, [[(r + 2 * p) % 8 for p in range(3)] for r in range(W)]):
        assert np.array_equal(run_copyin(tide, plan, bshards, shard_offsets=offs), bwant), offs


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_copyin_full_size_bit_exact(tide, oracle_mod, name):
    """fp32 master shards of every rank at the full layer shapes -> the
    rank-major bf16 buffer, every element, in the default launch options."""
    import os

    import torch

    w = synth.workload(name)
    print(f"\n[copy-in full-size] {name}", flush=True)
    plan = tide.Plan(w.world, w.shapes)
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.device_seed(w.index, 2000))
    params = [torch.randn(s, generator=g, device="cuda", dtype=torch.float32) * w.sigma for s in w.shapes]
    shards = []
    for r in range(w.world):
        row = []
        for p, s in enumerate(w.shapes):
            R = plan.rows_per_rank[p]
            row.append(params[p][min(r * R, s[0]):min((r + 1) * R, s[0])])
        shards.append(row)
    rm = torch.empty(w.world * plan.shard_elems, dtype=torch.bfloat16, device="cuda")
    tide.allgather_copyin(plan, shards, rm)
    torch.cuda.synchronize()
    got = gpu_util.bf16_bits(rm)
    host = [[t.cpu().numpy() for t in row] for row in shards]
    want = oracle_mod.copyin(w.world, w.shapes, host, nthreads=min(16, os.cpu_count() or 1))
    assert np.array_equal(got, want)
    print(f"[copy-in full-size] {name}: bit-exact", flush=True)


def test_registered_calls_match_the_oracle(tide, oracle_mod):
    """The *_call variants (tensors checked and pointers marshalled once)
    launch the same work: repeated launches give the oracle's bits."""
    import torch

    rng = np.random.default_rng(22)
    W = 8
    shapes = [(W * 30 + 5, 64), (9,), (W * 4, 1000)]
    grads_h = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    X = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    plan = tide.Plan(W, shapes)
    grads = [[gpu_util.to_device_bf16(g).view(s) for g, s in zip(row, shapes)] for row in grads_h]
    outs = [torch.empty(plan.shard_elems, dtype=torch.float32, device="cuda") for _ in range(W)]
    rm = torch.empty(W * plan.shard_elems, dtype=torch.bfloat16, device="cuda")
    params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    shards = [[torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in row]
              for row in oracle_pins.shards_of(W, shapes, X)]
    rs = tide.reduce_scatter_call(plan, grads, outs)
    ci = tide.allgather_copyin_call(plan, shards, rm)
    co = tide.allgather_copyout_call(plan, rm, params)
    want = oracle_mod.rs_local(W, shapes, grads_h)
    for _ in range(3):
        rs()
        ci()
        co()
        torch.cuda.synchronize()
        for r in range(W):
            gpu_util.assert_same_f32(outs[r].cpu().numpy(), want[r], f"rank {r}")
        for p in range(len(shapes)):
            assert np.array_equal(gpu_util.bf16_bits(params[p]).reshape(shapes[p]),
                                  oracle_mod.cast_bf16(X[p]).reshape(shapes[p]))
