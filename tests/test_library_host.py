"""Host-side checks of the HIP library (no GPU needed): it loads, exports
every symbol the header declares, its planner agrees with the oracle's, its
segment table describes exactly the oracle's result, and argument errors are
reported before any device work."""
import os
import re
import subprocess

import numpy as np
import pytest

import synth

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tide():
    from param_collectives_amd import tide

    return tide


def header_functions():
    text = open(os.path.join(ROOT, "include", "tide.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tide_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(tide):
    declared = header_functions()
    assert declared == sorted(tide.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", tide.LIBRARY], check=True, capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for name in declared:
        assert hasattr(tide.lib, name)


def test_library_has_no_oracle_dependency(tide):
    out = subprocess.run(["ldd", tide.LIBRARY], check=True, capture_output=True, text=True).stdout
    assert "oracle" not in out
    syms = subprocess.run(["nm", "-D", tide.LIBRARY], check=True, capture_output=True, text=True).stdout
    assert "oracle_" not in syms


CASES = [
    (4, oracle_pins.TINY_SHAPES),
    (8, [(4096, 4096), (1024, 4096), (4096,)]),
    (8, [(6, 5120), (5120,), (13824, 5120)]),
    (1, [(5, 3), (7,)]),
    (3, [(0, 4), (2, 0), (1,), (10, 1, 3)]),
    (256, [(300, 2), (1,)]),
]


def test_sizes_whose_byte_offsets_overflow_are_a_range_error(tide):
    # W * S elements must stay within 2^61 so that fp32 byte offsets fit int64
    with pytest.raises(tide.TideError) as e:
        tide.Plan(4, [(2**59 + 4,)])
    assert _status(e) == -2
    with pytest.raises(tide.TideError) as e:
        tide.Plan(1, [(2**60,), (2**60,)])
    assert _status(e) == -2


@pytest.mark.parametrize("world,shapes", CASES)
def test_layout_matches_oracle(tide, oracle_mod, world, shapes):
    plan = tide.Plan(world, shapes)
    geo = oracle_mod.plan(world, shapes)
    assert list(plan.rows_per_rank) == list(geo["R"])
    assert list(plan.shard_offset) == list(geo["o"])
    assert plan.shard_elems == geo["S"]


@pytest.mark.parametrize("world,shapes", CASES)
def test_exported_sizes_match_oracle(tide, oracle_mod, world, shapes):
    """The element counts the binding sizes its buffers by come from the
    library (tide_plan_sizes), and they are the oracle's: D_p*K_p per
    parameter, n_real(p, r) per rank's local shard."""
    plan = tide.Plan(world, shapes)
    geo = oracle_mod.plan(world, shapes)
    assert plan.numel == [int(d * k) for d, k in zip(geo["D"], geo["K"])]
    assert plan.n_real == [[int(geo["n_real"][p, r]) for p in range(len(shapes))] for r in range(world)]
    # either output may be omitted
    import ctypes

    buf = np.full(world * len(shapes), -7, dtype=np.int64)
    assert tide.lib.tide_plan_sizes(plan.handle, None, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))) == 0
    assert buf.reshape(world, -1).tolist() == plan.n_real
    assert tide.lib.tide_plan_sizes(plan.handle, None, None) == 0
    assert tide.lib.tide_plan_sizes(None, None, None) == -1


def test_binding_holds_no_layout_arithmetic():
    """The binding marshals: the shard geometry (rows per rank, real rows of a
    shard) is read from the library, never recomputed in Python."""
    src = open(os.path.join(ROOT, "param_collectives_amd", "tide.py")).read()
    assert "tide_plan_sizes" in src and "tide_plan_layout" in src
    for pattern in (r"\bmin\(", r"\bmax\(0", r"np\.prod", r"// ?s\[0\]", r"- ?r ?\*"):
        assert not re.search(pattern, src), pattern


@pytest.mark.parametrize("world,shapes", CASES)
def test_segments_describe_the_oracle_layout(tide, oracle_mod, world, shapes):
    """Each (rank, parameter) pair's real part is one sum segment reading
    n_real elements at the owner's first row, and its padding one zero
    segment; copy-out segments move exactly the real elements."""
    plan = tide.Plan(world, shapes)
    geo = oracle_mod.plan(world, shapes)
    rs = plan.segments(0)
    co = plan.segments(1)
    assert np.all(rs[:, 5] > 0) and np.all(co[:, 5] > 0)
    for p in range(len(shapes)):
        for r in range(world):
            real = geo["n_real"][p, r]
            pad = geo["n"][p] - real
            sums = rs[(rs[:, 0] == 0) & (rs[:, 1] == p) & (rs[:, 2] == r)]
            zeros = rs[(rs[:, 0] == 1) & (rs[:, 1] == p) & (rs[:, 2] == r)]
            copies = co[(co[:, 2] == p) & (co[:, 4] == r * geo["n"][p])]
            if real:
                assert len(sums) == 1 and tuple(sums[0, 3:]) == (r * geo["n"][p], geo["o"][p], real)
                assert len(copies) == 1 and tuple(copies[0, 3:]) == (geo["rank_major_offset"][p, r],
                                                                    r * geo["R"][p] * geo["K"][p], real)
            else:
                assert len(sums) == 0
            if pad:
                assert len(zeros) == 1 and tuple(zeros[0, 4:]) == (geo["o"][p] + real, pad)
            else:
                assert len(zeros) == 0
    assert rs[:, 5].sum() == world * geo["S"]  # every output element written once
    assert co[:, 5].sum() == sum(int(np.prod(s)) for s in shapes)


def _emulate_rs(plan, grads_f32):
    """Walk the library's segment table on the CPU (rank order, fp32)."""
    W, S = plan.world, plan.shard_elems
    outs = [np.full(S, np.nan, dtype=np.float32) for _ in range(W)]
    for kind, p, r, so, do, n in plan.segments(0):
        if kind == 1:
            outs[r][do:do + n] = 0.0
        else:
            acc = grads_f32[0][p].reshape(-1)[so:so + n].copy()
            for u in range(1, W):
                acc = acc + grads_f32[u][p].reshape(-1)[so:so + n]
            outs[r][do:do + n] = acc
    return outs


def _emulate_pack(plan, grads_u):
    """Walk the library's stock-pack segment table on the CPU."""
    out = np.full(plan.world * plan.shard_elems, np.nan, dtype=np.float32)
    for kind, p, _, so, do, n in plan.segments(3):
        if kind == 1:
            out[do:do + n] = 0.0
        else:
            out[do:do + n] = oracle_pins.f32_from_bf16(grads_u[p]).reshape(-1)[so:so + n]
    return out


@pytest.mark.parametrize("world,shapes", CASES)
def test_pack_segments_describe_the_oracle_layout(tide, oracle_mod, world, shapes):
    """The stock pack writes each (rank, parameter) slot of the rank-major fp32
    buffer: the rank's rows of the parameter, then zeros for its padding."""
    plan = tide.Plan(world, shapes)
    geo = oracle_mod.plan(world, shapes)
    pk = plan.segments(3)
    assert np.all(pk[:, 5] > 0)
    for p in range(len(shapes)):
        for r in range(world):
            real = geo["n_real"][p, r]
            pad = geo["n"][p] - real
            slot = geo["rank_major_offset"][p, r]
            mine = pk[(pk[:, 1] == p) & (pk[:, 4] >= slot) & (pk[:, 4] < slot + geo["n"][p])]
            copies, zeros = mine[mine[:, 0] == 2], mine[mine[:, 0] == 1]
            assert len(copies) == (1 if real else 0) and len(zeros) == (1 if pad else 0)
            if real:
                assert tuple(copies[0, 3:]) == (r * geo["R"][p] * geo["K"][p], slot, real)
            if pad:
                assert tuple(zeros[0, 4:]) == (slot + real, pad)
    assert pk[:, 5].sum() == world * geo["S"]  # the whole packed buffer is written


def test_pack_table_walk_reproduces_oracle(tide, oracle_mod):
    rng = np.random.default_rng(6)
    for world, shapes in CASES[:5]:
        if sum(int(np.prod(s)) for s in shapes) > 10**6:
            continue
        plan = tide.Plan(world, shapes)
        grads_u = [oracle_pins.rand_bf16(rng, s) for s in shapes]
        want = oracle_mod.chunk_cat(world, shapes, grads_u)
        assert oracle_pins.same_bits(_emulate_pack(plan, grads_u), want)


def test_segment_table_walk_reproduces_oracle(tide, oracle_mod):
    rng = np.random.default_rng(5)
    for world, shapes in CASES[:5]:
        if sum(int(np.prod(s)) for s in shapes) > 10**6:
            continue
        plan = tide.Plan(world, shapes)
        grads = [[oracle_pins.rand_bf16(rng, s) for s in shapes] for _ in range(world)]
        want = oracle_mod.rs_local(world, shapes, grads)
        f32 = [[oracle_pins.f32_from_bf16(g) for g in row] for row in grads]
        got = _emulate_rs(plan, f32)
        for r in range(world):
            assert oracle_pins.same_bits(got[r], want[r])


# ------------------------------------------------------------ error paths


def _status(excinfo):
    return excinfo.value.status


def test_plan_create_rejects_bad_arguments(tide):
    with pytest.raises(tide.TideError) as e:
        tide.Plan(0, [(4,)])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(tide.MAX_WORLD + 1, [(4,)])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [()])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [(3, -2)])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [(2**40, 2**30)])
    assert _status(e) == -2
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [(4,)], chunk_elems=12)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [(4,)], wg_per_cu=-1)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        tide.Plan(2, [(4,)], flags=0x80)
    assert _status(e) == -1


# Host addresses that are never dereferenced: every call below must fail its
# argument checks before any device work.
FAKE = 0x7F0000000000


def test_reduce_scatter_argument_errors(tide):
    plan = tide.Plan(4, oracle_pins.TINY_SHAPES)
    W, P = 4, 4
    good_g = [FAKE + 0x1000 * i for i in range(W * P)]
    good_o = [FAKE + 0x100000 + 0x1000 * r for r in range(W)]
    cases = [
        (dict(accumulate=2), -1),
        (dict(accumulate=-1), -1),
        (dict(grad_ptrs=good_g[:5] + [0] + good_g[6:]), -1),
        (dict(grad_ptrs=good_g[:5] + [FAKE + 1] + good_g[6:]), -3),
        (dict(grad_ptrs=good_g[:5] + [FAKE + 2] + good_g[6:], f32=True), -3),
        (dict(out_ptrs=good_o[:2] + [0] + good_o[3:]), -1),
        (dict(out_ptrs=good_o[:2] + [FAKE + 2] + good_o[3:]), -3),
        (dict(out_ptrs=good_o[:2] + [FAKE + 2] + good_o[3:], f32=True, alpha=-3.0), -3),
    ]
    for kw, status in cases:
        args = dict(grad_ptrs=good_g, out_ptrs=good_o, alpha=1.0, accumulate=0, f32=False)
        args.update(kw)
        with pytest.raises(tide.TideError) as e:
            plan.reduce_scatter_local_raw(args["grad_ptrs"], args["out_ptrs"], args["alpha"], args["accumulate"],
                                          f32=args["f32"])
        assert _status(e) == status, kw
        assert tide.lib.tide_last_error()


def test_stock_pack_argument_errors(tide):
    plan = tide.Plan(4, oracle_pins.TINY_SHAPES)
    good = [FAKE + 0x1000 * i for i in range(4)]
    for grads, packed, status in [
        (good[:2] + [0] + good[3:], FAKE, -1),
        (good[:2] + [FAKE + 1] + good[3:], FAKE, -3),
        (good, 0, -1),
        (good, FAKE + 2, -3),
    ]:
        with pytest.raises(tide.TideError) as e:
            plan.stock_chunk_cat_raw(grads, packed)
        assert _status(e) == status
    # a parameter with no elements may be NULL; the call still fails on `packed`
    plan = tide.Plan(2, [(0, 4), (3,)])
    with pytest.raises(tide.TideError) as e:
        plan.stock_chunk_cat_raw([0, FAKE], FAKE + 1)
    assert _status(e) == -3


def test_copyout_argument_errors(tide):
    plan = tide.Plan(4, oracle_pins.TINY_SHAPES)
    good_p = [FAKE + 0x1000 * i for i in range(4)]
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyout_raw(FAKE, good_p[:1] + [0] + good_p[2:])
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyout_raw(FAKE, good_p[:1] + [FAKE + 3] + good_p[2:])
    assert _status(e) == -3
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyout_raw(FAKE + 1, good_p)
    assert _status(e) == -3
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyout_raw(0, good_p)
    assert _status(e) == -1


def test_raw_calls_check_pointer_counts(tide):
    # the library reads exactly W*P, W or P addresses: a short list is refused
    # before the call
    plan = tide.Plan(4, oracle_pins.TINY_SHAPES)
    g = [FAKE + 0x1000 * i for i in range(16)]
    o = [FAKE + 0x100000 + 0x1000 * r for r in range(4)]
    calls = [
        lambda: plan.reduce_scatter_local_raw(g[:15], o),
        lambda: plan.reduce_scatter_local_raw(g, o[:3]),
        lambda: plan.reduce_scatter_local_raw(g + [FAKE], o, f32=True),
        lambda: plan.stock_chunk_cat_raw(g[:3], FAKE),
        lambda: plan.allgather_copyout_raw(FAKE, g[:5]),
        lambda: plan.allgather_copyin_raw(g[:12], tide.DTYPE_F32, FAKE),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="addresses"):
            call()


def test_destroyed_plan_is_rejected(tide):
    plan = tide.Plan(2, [(4,)])
    handle = plan.handle
    plan.destroy()
    import ctypes

    R = (ctypes.c_int64 * 1)()
    assert tide.lib.tide_plan_layout(handle, R, None, None) == -1
    assert b"destroyed" in tide.lib.tide_last_error()
    tide.lib.tide_plan_destroy(handle)  # a second destroy is harmless
    tide.lib.tide_plan_destroy(None)


def test_options_round_trip_and_validation(tide):
    plan = tide.Plan(8, [(64, 64)], cu_budget=16, wg_per_cu=2, chunk_elems=1024, flags=tide.FLAG_CACHED_LOADS)
    assert plan.options(0) == {"cu_budget": 16, "wg_per_cu": 2, "chunk_elems": 1024, "flags": 1, "wave_chunks": 64}
    assert plan.options(1) == {"cu_budget": 16, "wg_per_cu": 2, "chunk_elems": 1024, "flags": 1, "wave_chunks": 64}
    before = plan.segments(0).copy()
    plan.set_options(chunk_elems=8)
    assert plan.options()["chunk_elems"] == 8
    assert np.array_equal(plan.segments(0), before)  # knobs never change the work
    with pytest.raises(tide.TideError):
        plan.set_options(chunk_elems=7)
    with pytest.raises(tide.TideError):
        plan.set_options(wg_per_cu=1000)
    with pytest.raises(tide.TideError):
        plan.set_options(chunk_elems=2**28 + 8)
    plan.set_options(chunk_elems=2**28)
    # zero fields take each operation's default (cu_budget resolves on a device)
    with pytest.raises(tide.TideError):
        plan.set_options(wave_chunks=-1)
    with pytest.raises(tide.TideError):
        plan.set_options(wave_chunks=2**30 + 1)
    plan.set_options(wave_chunks=3)
    assert plan.options(2)["wave_chunks"] == 3
    plan.set_options()
    assert plan.options(0) == {"cu_budget": 0, "wg_per_cu": 1, "chunk_elems": 1024, "flags": 0, "wave_chunks": 64}
    assert plan.options(1) == {"cu_budget": 0, "wg_per_cu": 1, "chunk_elems": 4096, "flags": 0, "wave_chunks": 64}
    assert plan.options(2) == {"cu_budget": 0, "wg_per_cu": 1, "chunk_elems": 4096, "flags": 0, "wave_chunks": 64}
    assert plan.options(3) == {"cu_budget": 0, "wg_per_cu": 1, "chunk_elems": 2048, "flags": 0, "wave_chunks": 64}
    assert plan.options(4) == {"cu_budget": 0, "wg_per_cu": 1, "chunk_elems": 256, "flags": 0, "wave_chunks": 64}
    assert np.array_equal(plan.segments(4), plan.segments(0))
    for bad in (-1, 5):
        with pytest.raises(tide.TideError) as e:
            plan.options(bad)
        assert _status(e) == -1
        with pytest.raises(tide.TideError) as e:
            plan.segments(bad)
        assert _status(e) == -1


def _launch_groups(op, segs, cb, waves, wave_chunks):
    """First chunks of the launch groups, re-derived from the segment table:
    in a reduce-scatter (ops 0 and 4), a run of segments with one destination
    rank (column 2) of at least one round opens a group when it starts more
    than waves/64 chunks off the current group's round boundaries and that
    group holds wave_chunks/2 rounds; other operations are one group."""
    if op not in (0, 4):
        return [0]
    tol = max(1, waves // 64)
    min_group = waves * max(1, wave_chunks // 2)
    cuts = [0]
    i = 1
    while i < len(segs):
        if segs[i, 2] == segs[i - 1, 2]:
            i += 1
            continue
        j = i + 1
        while j < len(segs) and segs[j, 2] == segs[i, 2]:
            j += 1
        c, run = int(cb[i]), int(cb[j] - cb[i])
        phase = (c - cuts[-1]) % waves
        if tol < phase < waves - tol and run >= waves and c - cuts[-1] >= min_group:
            cuts.append(c)
        i = j
    return cuts


def _check_launches(plan, op, L, waves, wave_chunks):
    """The launch table of one operation against its definition: consecutive
    chunk ranges covering every chunk; within each launch group, equal whole
    rounds per launch but the group's last, at most wave_chunks rounds each;
    and the segment range of each launch found from the chunk table of the
    plan's segments.  Returns the group starts."""
    segs = plan.segments(op)
    chunk = plan.options(op)["chunk_elems"]
    cb = np.concatenate([[0], np.cumsum(-(-segs[:, 5] // chunk))])
    nchunks = int(cb[-1])
    assert L[0, 0] == 0 and L[-1, 1] == nchunks
    assert np.array_equal(L[1:, 0], L[:-1, 1])
    cuts = _launch_groups(op, segs, cb, waves, wave_chunks)
    assert set(cuts) <= set(L[:, 0].tolist())
    bounds = cuts + [nchunks]
    for g0, g1 in zip(bounds[:-1], bounds[1:]):
        G = L[(L[:, 0] >= g0) & (L[:, 0] < g1)]
        assert G[0, 0] == g0 and G[-1, 1] == g1
        lens = G[:, 1] - G[:, 0]
        assert np.all(lens[:-1] == lens[0]) and 0 < lens[-1] <= lens[0]
        assert lens[0] % waves == 0 or len(G) == 1
        assert np.all(lens <= wave_chunks * waves)
        rounds = -(-(g1 - g0) // waves)
        assert len(G) == -(-rounds // wave_chunks)
    for first, end, seg, seg_end, g in L:
        assert cb[seg] <= first < cb[seg + 1]
        assert cb[seg_end - 1] <= end - 1 < cb[seg_end]
        assert g == min(waves // 4, -(-(end - first) // 4))
    return cuts


def test_launch_split(tide):
    w = synth.workload("llama3.1-8b-layer")
    plan = tide.Plan(w.world, w.shapes)
    L = plan.launches(0, cu_count=256)
    # every rank owns 2 mod 1024 chunks: one group
    assert _check_launches(plan, 0, L, 1024, 64) == [0]
    # 213,008 chunks are 209 rounds of 1024 waves: four launches of 53 rounds, the last shorter
    assert len(L) == 4
    assert list(L[:, 1] - L[:, 0]) == [53 * 1024] * 3 + [213008 - 3 * 53 * 1024]
    for op in range(5):
        _check_launches(plan, op, plan.launches(op, cu_count=256), 1024, 64)
    # the Qwen3 layer's ranks own 76,068 chunks (292 mod 1024): every rank's
    # shard opens a group, split into launches of 38 and 36 rounds; each
    # launch touches a few hundred of its segments
    q = synth.workload("qwen3-30b-a3b-moe-layer")
    qplan = tide.Plan(q.world, q.shapes)
    QL = qplan.launches(0, cu_count=256)
    assert _check_launches(qplan, 0, QL, 1024, 64) == [r * 76068 for r in range(8)]
    assert len(QL) == 16 and list(QL[:2, 1] - QL[:2, 0]) == [38 * 1024, 76068 - 38 * 1024]
    assert np.all(QL[:, 3] - QL[:, 2] < 400)
    # the Wan2.2 block: one group per rank shard for the reduce-scatter, one
    # group for the copy-out
    v = synth.workload("wan2.2-dit-block")
    vplan = tide.Plan(v.world, v.shapes)
    assert len(_check_launches(vplan, 0, vplan.launches(0, cu_count=256), 1024, 64)) == 8
    assert len(_check_launches(vplan, 1, vplan.launches(1, cu_count=256), 1024, 64)) == 1
    # a small grid, three rounds per launch, a short last launch
    rng = np.random.default_rng(5)
    shapes = [(int(rng.integers(1, 40)), int(rng.integers(1, 70))) for _ in range(30)]
    small = tide.Plan(3, shapes, cu_budget=2, wg_per_cu=1, chunk_elems=16, wave_chunks=3)
    for op in range(5):
        _check_launches(small, op, small.launches(op), 8, 3)
    assert len(small.launches(0)) > 3
    # ranks of a few rounds each at an odd phase are grouped, not cut one by one
    many = tide.Plan(64, w.shapes)
    cuts = _check_launches(many, 0, many.launches(0, cu_count=256), 1024, 64)
    assert len(cuts) < 8


def test_launches_need_a_cu_count_until_bound(tide):
    plan = tide.Plan(2, [(64, 64)])
    with pytest.raises(tide.TideError) as e:
        plan.launches(0)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        plan.launches(0, cu_count=-1)
    assert _status(e) == -1
    assert len(plan.launches(0, cu_count=4)) == 1
    empty = tide.Plan(2, [(0, 4)])
    assert empty.launches(0, cu_count=4).shape == (0, 5)


def test_launch_table_capacity(tide):
    """A table shorter than the launch count gets the first launches and the
    full count."""
    import ctypes

    q = synth.workload("qwen3-30b-a3b-moe-layer")
    plan = tide.Plan(q.world, q.shapes)
    full = plan.launches(0, cu_count=256)
    table = np.full((3, 5), -7, dtype=np.int64)
    count = ctypes.c_int64(-1)
    st = tide.lib.tide_plan_launches(plan.handle, 0, 256, table.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 2,
                                     ctypes.byref(count))
    assert st == 0 and count.value == len(full) == 16
    assert np.array_equal(table[:2], full[:2]) and np.all(table[2] == -7)


def test_too_many_chunks_is_a_range_error(tide):
    with pytest.raises(tide.TideError) as e:
        tide.Plan(1, [(2**34,)], chunk_elems=8)
    assert _status(e) == -2
    tide.Plan(1, [(2**33,)], chunk_elems=8)  # exactly 2^30 chunks: the limit
    with pytest.raises(tide.TideError) as e:
        tide.Plan(1, [(2**33 + 8,)], chunk_elems=8)
    assert _status(e) == -2
    plan = tide.Plan(1, [(2**34,)])  # 2^23 chunks of the default size (2048 elements for W <= 3)
    before = plan.options(0)
    assert before["chunk_elems"] == 2048
    with pytest.raises(tide.TideError) as e:
        plan.set_options(chunk_elems=8)
    assert _status(e) == -2
    assert plan.options(0) == before  # unchanged after the failed call


@pytest.mark.parametrize("world,shapes", CASES)
def test_copyin_segments_describe_the_oracle_layout(tide, oracle_mod, world, shapes):
    """Each (rank, parameter) slot of the rank-major buffer is one copy segment
    of the rank's real elements followed by one zero segment of padding."""
    plan = tide.Plan(world, shapes)
    geo = oracle_mod.plan(world, shapes)
    ci = plan.segments(2)
    P = len(shapes)
    assert np.all(ci[:, 5] > 0)
    for p in range(P):
        for r in range(world):
            real = geo["n_real"][p, r]
            pad = geo["n"][p] - real
            slot = geo["rank_major_offset"][p, r]
            mine = ci[ci[:, 1] == r * P + p]
            copies, zeros = mine[mine[:, 0] == 2], mine[mine[:, 0] == 1]
            assert len(copies) == (1 if real else 0) and len(zeros) == (1 if pad else 0)
            if real:
                assert tuple(copies[0, 3:]) == (0, slot, real)
            if pad:
                assert tuple(zeros[0, 4:]) == (slot + real, pad)
    assert ci[:, 5].sum() == world * geo["S"]  # the whole rank-major buffer is written


def test_copyin_argument_errors(tide):
    plan = tide.Plan(4, oracle_pins.TINY_SHAPES)
    good = [FAKE + 0x1000 * i for i in range(16)]
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good[:3] + [0] + good[4:], tide.DTYPE_F32, FAKE)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good[:3] + [FAKE + 2] + good[4:], tide.DTYPE_F32, FAKE)
    assert _status(e) == -3
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good, 7, FAKE)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good, tide.DTYPE_BF16, 0)
    assert _status(e) == -1
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good, tide.DTYPE_BF16, FAKE + 1)
    assert _status(e) == -3
    # rank 3 holds nothing of parameter 3 ([3,3,4] with W = 4): its shard may be NULL,
    # but the call still fails (later) on the misaligned buffer
    with pytest.raises(tide.TideError) as e:
        plan.allgather_copyin_raw(good[:15] + [0], tide.DTYPE_BF16, FAKE + 1)
    assert _status(e) == -3


def test_instrument_argument_errors(tide):
    """Checks of the interference instruments that fail before any device
    call (no GPU is touched)."""
    import ctypes

    lib = tide.lib
    vp = ctypes.c_void_p
    assert lib.tide_probe_launch(None, 1, 0, 0, None) == -1
    assert lib.tide_probe_launch(vp(FAKE + 2), 1, 0, 0, None) == -3
    assert lib.tide_probe_launch(vp(FAKE), 0, 0, 0, None) == -1
    assert lib.tide_probe_launch(vp(FAKE), 65537, 0, 0, None) == -1
    assert lib.tide_probe_launch(vp(FAKE), 4, 0, -1, None) == -1
    assert lib.tide_probe_launch(vp(FAKE), 4, 0, 10**9 + 1, None) == -1
    assert b"hold_ns" in lib.tide_last_error()
    f = ctypes.c_float
    assert lib.tide_victim_axpb(vp(FAKE), vp(FAKE), -1, f(1), f(0), None) == -1
    assert lib.tide_victim_axpb(None, vp(FAKE), 5, f(1), f(0), None) == -1
    assert lib.tide_victim_axpb(vp(FAKE + 2), vp(FAKE), 5, f(1), f(0), None) == -3
    assert lib.tide_victim_axpb(None, None, 0, f(1), f(0), None) == 0  # nothing to do
    assert lib.tide_stream_create(None, 0, None) == -1
    assert lib.tide_stream_destroy(None) == 0


def test_probe_record_decoding(tide):
    """The probe's register fields, decoded from hand-built records."""
    hw = (5 << 0) | (2 << 4) | (1 << 6) | (11 << 8) | (1 << 12) | (3 << 13)
    rec = np.array([7, hw, 6, 0, 0xFFFFFFFF, 1, 5, 2], dtype=np.uint32)
    d = tide.decode_probe(rec)
    assert (d["block"][0], d["wave"][0], d["simd"][0], d["cu"][0], d["sh"][0], d["se"][0], d["xcc"][0]) == \
        (7, 5, 2, 11, 1, 3, 6)
    assert d["ok"][0] and d["entry"][0] == 2**33 - 1 and d["exit"][0] == 2**33 + 5


def test_paths_need_a_call_first(tide):
    """tide_plan_paths reports the latest call's tables: before any call it is
    an argument error (host only), as are a bad op and a null output."""
    import ctypes

    plan = tide.Plan(4, [(8, 3)])
    out = (ctypes.c_int64 * 4)()
    assert tide.lib.tide_plan_paths(plan.handle, 0, out) == -1
    assert "no call" in tide.lib.tide_last_error().decode()
    assert tide.lib.tide_plan_paths(plan.handle, 5, out) == -1
    assert tide.lib.tide_plan_paths(plan.handle, 0, None) == -1
    assert tide.lib.tide_plan_paths(None, 0, out) == -1


def test_readme_example_uses_the_binding_as_it_is(tide):
    """The README's Python example compiles, and every binding name it calls
    exists with the keyword arguments it passes."""
    import inspect

    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")).read()
    code = re.search(r"```python\n(.*?)```", src, re.S).group(1)
    compile(code, "README.md", "exec")
    for name in re.findall(r"tide\.(\w+)\(", code):
        assert hasattr(tide, name), name
    assert "alpha" in inspect.signature(tide.reduce_scatter_call).parameters
