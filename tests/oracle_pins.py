"""Checks that pin the CPU oracle to things other than itself.

Each check takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with:
  * values worked by hand from the definitions (tests/golden/*.txt);
  * an independent brute-force route to the same result: the stock FSDP2
    path that TIDE replaces ("The Endgame of FSDP Communication", Section
    2.1, Equation 3) -- zero-pad each gradient to W*R_p rows, widen to
    fp32, pack rank-major by destination, then reduce-scatter the packed
    buffers -- whose result the pages say TIDE leaves unchanged;
  * closed forms (exact integer sums, W*x, one-hot ranks, subnormals);
  * invariants (row ownership partitions, landing tiles, round trips);
  * the pages' error bound against an fp64 sum (Section 4.3) and Higham's
    recursive-summation bound.
The same checks run against deliberately broken builds of the oracle in
test_oracle_mutants.py, each of which must fail at least one of them.
"""
import numpy as np

from tests import goldens

TINY_SHAPES = [(7, 5), (16,), (33, 8), (3, 3, 4)]


def f32_from_bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rand_bf16(rng, shape, scale=1.0):
    v = (rng.standard_normal(int(np.prod(shape, dtype=np.int64))) * scale).astype(np.float32)
    # truncate to bf16 (any bf16 values will do as inputs)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16).reshape(shape)


def random_case(rng, W, P, max_rows=13, max_k=7):
    shapes = []
    for _ in range(P):
        nd = int(rng.integers(1, 4))
        dims = [int(rng.integers(0, max_rows + 1))] + [int(rng.integers(0, max_k + 1)) for _ in range(nd - 1)]
        shapes.append(tuple(dims))
    return shapes


# ---------------------------------------------------------------- planner


def check_tiny_plan_golden(orc):
    g = goldens.read("tiny_plan.txt")
    W = int(g["world"][0][0])
    shapes = [tuple(goldens.ints(s)) for s in g["shape"]]
    geo = orc.plan(W, shapes)
    for key in ("D", "K", "R", "n", "o"):
        assert list(geo[key]) == goldens.ints(g[key][0]), key
    assert geo["S"] == int(g["S"][0][0])
    for key in ("n_real", "rank_major_offset", "landing_offset"):
        for row in g[key]:
            p, vals = int(row[0]), goldens.ints(row[1:])
            assert list(geo[key][p]) == vals, (key, p)


def check_plan_invariants(orc, seed=1):
    rng = np.random.default_rng(seed)
    for W in (1, 2, 3, 4, 5, 8):
        for _ in range(20):
            shapes = random_case(rng, W, int(rng.integers(1, 7)))
            geo = orc.plan(W, shapes)
            P = len(shapes)
            S = geo["S"]
            landing_cover = np.zeros(W * S, dtype=np.int64)
            rank_major_cover = np.zeros(W * S, dtype=np.int64)
            for p in range(P):
                D = shapes[p][0]
                K = int(np.prod(shapes[p][1:], dtype=np.int64))
                assert geo["D"][p] == D and geo["K"][p] == K
                # rows are handed out in rank order in blocks of R: every rank
                # before the last real one holds R rows, later ranks hold none
                if K > 0:
                    assert np.all(geo["n_real"][p] % K == 0)
                    rows = geo["n_real"][p] // K
                    assert np.all((rows >= 0) & (rows <= geo["R"][p]))
                    short = np.nonzero(rows < geo["R"][p])[0]
                    if short.size:
                        assert np.all(rows[short[0] + 1:] == 0), (shapes, p)
                    assert rows.sum() == D
                else:
                    assert np.all(geo["n_real"][p] == 0)
                assert geo["n_real"][p].sum() == D * K
                assert geo["R"][p] * W >= D and (geo["R"][p] - 1) * W < max(D, 1)
                for r in range(W):
                    lo = geo["landing_offset"][p, r]
                    landing_cover[lo:lo + geo["n"][p]] += 1
                    rm = geo["rank_major_offset"][p, r]
                    rank_major_cover[rm:rm + geo["n"][p]] += 1
                    # the rank-major slot of (p, r) lies inside rank r's S-element shard
                    assert r * S <= rm and rm + geo["n"][p] <= (r + 1) * S
                # parameter-major: p's W shards are contiguous, in rank order
                assert np.all(np.diff(geo["landing_offset"][p]) == geo["n"][p])
            # both buffers are tiled exactly once by the (p, r) slots
            assert np.all(landing_cover == 1) and np.all(rank_major_cover == 1)


def check_landing_is_padded_parameter(orc, seed=2):
    """Scattering pack()'s rank-major slots to their landing offsets gives each
    parameter contiguously (followed by its zero padding), as Equation 2 says
    the compute kernels need it."""
    rng = np.random.default_rng(seed)
    for W in (1, 3, 4, 8):
        shapes = random_case(rng, W, 5)
        X = [rand_bf16(rng, s) for s in shapes]
        geo = orc.plan(W, shapes)
        rm = orc.pack(W, shapes, X)
        arena = np.full(W * geo["S"], 0xFFFF, dtype=np.uint16)
        for p in range(len(shapes)):
            for r in range(W):
                a, b = geo["rank_major_offset"][p, r], geo["landing_offset"][p, r]
                arena[b:b + geo["n"][p]] = rm[a:a + geo["n"][p]]
        for p in range(len(shapes)):
            base = geo["landing_offset"][p, 0]
            numel = X[p].size
            assert np.array_equal(arena[base:base + numel], X[p].reshape(-1))
            assert np.all(arena[base + numel:base + W * geo["n"][p]] == 0)


# --------------------------------------------------------- reduce-scatter


def stock_fsdp2_pack(W, shapes, grads_u):
    """Stock FSDP2's packed fp32 input of one source rank: every parameter
    zero-padded to W*R_p rows and widened (fp32 taken as is), then rank r's
    rows of every parameter concatenated, ranks one after the other."""
    pieces_by_dest = [[] for _ in range(W)]
    for p, shape in enumerate(shapes):
        D = shape[0]
        K = int(np.prod(shape[1:], dtype=np.int64))
        R = -(-D // W)
        a = np.asarray(grads_u[p])
        g = (a.astype(np.float32) if a.dtype == np.float32 else f32_from_bf16(a)).reshape(D, K)
        padded = np.zeros((W * R, K), dtype=np.float32)
        padded[:D] = g
        for r in range(W):
            pieces_by_dest[r].append(padded[r * R:(r + 1) * R].reshape(-1))
    return np.concatenate([np.concatenate(pc) if pc else np.zeros(0, np.float32) for pc in pieces_by_dest])


def stock_fsdp2_reduce_scatter(W, shapes, grads):
    """Brute force by the stock path: pad, widen, pack rank-major, then sum
    the W packed buffers in rank order and give rank r its S-element slice."""
    packed = [stock_fsdp2_pack(W, shapes, grads[u]) for u in range(W)]
    total = packed[0].copy()
    for u in range(1, W):
        total = total + packed[u]
    S = total.size // W
    return [total[r * S:(r + 1) * S] for r in range(W)]


def same_bits(a, b):
    """Bitwise equal, except that any NaN matches any NaN."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    nan = np.isnan(a)
    return bool(np.array_equal(nan, np.isnan(b)) and np.array_equal(a.view(np.uint32)[~nan],
                                                                     b.view(np.uint32)[~nan]))


def check_rs_worked_golden(orc):
    g = goldens.read("rs_worked.txt")
    W = int(g["world"][0][0])
    shapes = [tuple(goldens.ints(s)) for s in g["shape"]]
    grads = [[None] for _ in range(W)]
    for row in g["grad"]:
        grads[int(row[0])][0] = goldens.hex16(row[1:]).reshape(shapes[0])
    out = orc.rs_local(W, shapes, grads)
    for row in g["out"]:
        r = int(row[0])
        for e, tok in enumerate(row[1:]):
            if tok == "nan":
                assert np.isnan(out[r][e]), (r, e)
            else:
                assert out[r].view(np.uint32)[e] == int(tok, 16), (r, e, hex(out[r].view(np.uint32)[e]), tok)


def check_rs_matches_stock_path(orc, seed=3):
    rng = np.random.default_rng(seed)
    cases = [(4, TINY_SHAPES)]
    for W in (1, 2, 3, 4, 8):
        for _ in range(6):
            cases.append((W, random_case(rng, W, int(rng.integers(1, 6)))))
    cases.append((8, [(3, 5), (0, 4), (9,), (1,), (17, 1, 3)]))  # D < W, D = 0, K = 1
    for W, shapes in cases:
        grads = [[rand_bf16(rng, s, scale=float(rng.choice([1e-3, 1.0, 1e3]))) for s in shapes] for _ in range(W)]
        got = orc.rs_local(W, shapes, grads)
        want = stock_fsdp2_reduce_scatter(W, shapes, grads)
        for r in range(W):
            assert same_bits(got[r], want[r]), (W, shapes, r)


def check_rs_w1_identity(orc, seed=4):
    rng = np.random.default_rng(seed)
    shapes = [(5, 3), (8,), (1, 1, 2)]
    grads = [[rand_bf16(rng, s) for s in shapes]]
    out = orc.rs_local(1, shapes, grads)[0]
    assert same_bits(out, np.concatenate([f32_from_bf16(g).reshape(-1) for g in grads[0]]))


def check_rs_integer_inputs_exact(orc, seed=5):
    """Integer-valued inputs with exactly representable sums: the fp32 result
    is the exact integer sum (the pages' bit-exact integer check)."""
    rng = np.random.default_rng(seed)
    for W in (2, 3, 8):
        shapes = [(W * 3 + 1, 4), (7,), (2, 5)]
        ints = [[rng.integers(-256, 257, size=s) for s in shapes] for _ in range(W)]
        grads = [[(np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16) for v in row]
                 for row in ints]
        got = orc.rs_local(W, shapes, grads)
        geo = orc.plan(W, shapes)
        for r in range(W):
            for p, s in enumerate(shapes):
                K = int(np.prod(s[1:], dtype=np.int64))
                R = geo["R"][p]
                exact = np.zeros(R * K, dtype=np.int64)
                rows = np.arange(r * R, min((r + 1) * R, s[0]))
                for u in range(W):
                    exact[:rows.size * K] += ints[u][p].reshape(s[0], K)[rows].reshape(-1)
                seg = got[r][geo["o"][p]:geo["o"][p] + R * K]
                assert np.array_equal(seg.astype(np.int64), exact) and np.all(seg == exact.astype(np.float32))


def check_rs_identical_ranks(orc, seed=6):
    """W copies of x sum to W*x exactly (W*x needs at most 11 significant bits)."""
    rng = np.random.default_rng(seed)
    for W in (2, 3, 5, 8):
        shapes = [(2 * W + 1, 3), (W,)]
        base = [rand_bf16(rng, s) for s in shapes]
        base = [np.where((b & 0x7F80) == 0x7F80, np.uint16(0x3F80), b) for b in base]  # finite only
        got = orc.rs_local(W, shapes, [base] * W)
        geo = orc.plan(W, shapes)
        for r in range(W):
            for p, s in enumerate(shapes):
                K = int(np.prod(s[1:], dtype=np.int64))
                n_real = geo["n_real"][p, r]
                first = r * geo["R"][p] * K
                x = f32_from_bf16(base[p]).reshape(-1)[first:first + n_real]
                seg = got[r][geo["o"][p]:geo["o"][p] + n_real]
                assert same_bits(seg, np.float32(W) * x)


def check_rs_one_hot_rank(orc, seed=7):
    rng = np.random.default_rng(seed)
    W = 4
    shapes = TINY_SHAPES
    for v in range(W):
        grads = [[np.zeros(s, dtype=np.uint16) for s in shapes] for _ in range(W)]
        grads[v] = [rand_bf16(rng, s) for s in shapes]
        got = orc.rs_local(W, shapes, grads)
        alone = orc.rs_local(W, shapes, [grads[v] if u == 0 else [np.zeros(s, np.uint16) for s in shapes]
                                         for u in range(W)])
        geo = orc.plan(W, shapes)
        for r in range(W):
            for p, s in enumerate(shapes):
                K = int(np.prod(s[1:], dtype=np.int64))
                n_real = geo["n_real"][p, r]
                first = r * geo["R"][p] * K
                x = f32_from_bf16(grads[v][p]).reshape(-1)[first:first + n_real]
                seg = got[r][geo["o"][p]:geo["o"][p] + n_real]
                assert np.array_equal(seg, x)  # numeric equality (+0 vs -0 aside)
            assert np.array_equal(got[r], alone[r])


def check_rs_sum_over_ranks(orc, seed=8):
    """For integer inputs: the sum of all outputs equals the sum of all inputs."""
    rng = np.random.default_rng(seed)
    for W in (3, 4, 8):
        shapes = random_case(rng, W, 5)
        ints = [[rng.integers(-100, 101, size=s) for s in shapes] for _ in range(W)]
        grads = [[(np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16) for v in row]
                 for row in ints]
        got = orc.rs_local(W, shapes, grads)
        total_in = sum(int(np.sum(v)) for row in ints for v in row)
        total_out = sum(int(np.sum(o.astype(np.int64))) for o in got)
        assert total_in == total_out


def check_rs_fp64_bounds(orc, seed=9):
    """|out - fp64 sum| <= gamma_{W-1} * sum |g| (recursive summation), and the
    pages' 1e-5 * max(1, ||y_ref||_inf) bound."""
    rng = np.random.default_rng(seed)
    for W in (2, 4, 8):
        shapes = [(W * 9 + 3, 17), (31,)]
        grads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
        got = orc.rs_local(W, shapes, grads)
        geo = orc.plan(W, shapes)
        u = 2.0 ** -24
        gamma = (W - 1) * u / (1 - (W - 1) * u)
        for r in range(W):
            for p, s in enumerate(shapes):
                K = int(np.prod(s[1:], dtype=np.int64))
                n_real = geo["n_real"][p, r]
                first = r * geo["R"][p] * K
                vals = np.stack([f32_from_bf16(grads[uu][p]).reshape(-1)[first:first + n_real].astype(np.float64)
                                 for uu in range(W)])
                exact = vals.sum(axis=0)
                seg = got[r][geo["o"][p]:geo["o"][p] + n_real].astype(np.float64)
                err = np.abs(seg - exact)
                assert np.all(err <= gamma * np.abs(vals).sum(axis=0))
                if n_real:
                    assert err.max() <= 1e-5 * max(1.0, np.abs(exact).max())


def check_rs_thread_invariance(orc, seed=10):
    rng = np.random.default_rng(seed)
    W = 8
    shapes = random_case(rng, W, 9, max_rows=40, max_k=9)
    grads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    one = orc.rs_local(W, shapes, grads, nthreads=1)
    for nt in (2, 3, 8):
        many = orc.rs_local(W, shapes, grads, nthreads=nt)
        for r in range(W):
            assert np.array_equal(one[r].view(np.uint32), many[r].view(np.uint32))


def check_rs_special_values(orc):
    W = 8
    shapes = [(8, 1)]
    qnan, inf, ninf, big, one = 0x7FC0, 0x7F80, 0xFF80, 0x7F7F, 0x3F80

    def run(col):
        grads = [[np.array([[col[u]]] * 8, dtype=np.uint16).reshape(8, 1)] for u in range(W)]
        return np.array([o[0] for o in orc.rs_local(W, shapes, grads)])

    assert np.all(np.isnan(run([one] * 7 + [qnan])))
    assert np.all(np.isnan(run([inf, ninf] + [one] * 6)))
    assert np.all(run([big] * 8) == np.inf)
    assert np.all(run([inf] + [one] * 7) == np.inf)
    sub = run([0x0001, 0x0001] + [0] * 6)
    assert np.all(sub.view(np.uint32) == 0x00020000)  # 2^-132: kept, not flushed
    negz = run([0x8000] * 8)
    assert np.all(negz.view(np.uint32) == 0x80000000)


def check_rs_padding_positive_zero(orc):
    W = 4
    shapes = [(5, 2), (1,), (0, 3)]
    grads = [[np.full(s, 0x8000 if u % 2 else 0xBF80, dtype=np.uint16) for s in shapes] for u in range(W)]
    got = orc.rs_local(W, shapes, grads)
    geo = orc.plan(W, shapes)
    for r in range(W):
        for p in range(len(shapes)):
            lo, hi = geo["o"][p] + geo["n_real"][p, r], geo["o"][p] + geo["n"][p]
            assert np.all(got[r][lo:hi].view(np.uint32) == 0)


def check_rs_linearity(orc, seed=11):
    """Inputs with disjoint supports: out(a + b) = out(a) + out(b) exactly (each
    element sums one non-zero value, the others are +0)."""
    rng = np.random.default_rng(seed)
    W = 3
    shapes = [(7, 3), (4,)]
    a = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    masks = [[rng.random(s) < 0.5 for s in shapes] for _ in range(W)]
    A = [[np.where(m, x, np.uint16(0)) for x, m in zip(ra, rm)] for ra, rm in zip(a, masks)]
    B = [[np.where(m, np.uint16(0), x) for x, m in zip(ra, rm)] for ra, rm in zip(a, masks)]
    # make the supports disjoint across ranks too: rank u keeps only elements with index % W == u
    def keep(t, u):
        flat = t.reshape(-1).copy()
        idx = np.arange(flat.size)
        flat[idx % W != u] = 0
        return flat.reshape(t.shape)
    A = [[keep(x, u) for x in A[u]] for u in range(W)]
    B = [[keep(x, u) for x in B[u]] for u in range(W)]
    AB = [[x | y for x, y in zip(A[u], B[u])] for u in range(W)]
    oa, ob, oab = (orc.rs_local(W, shapes, g) for g in (A, B, AB))
    for r in range(W):
        assert np.array_equal(oa[r] + ob[r], oab[r])


# ------------------------------------------------------------- copy-out


def stock_fsdp2_copyout(W, shapes, rank_major):
    """Brute force by the stock path: view the all-gather output as W rows of S,
    cut each parameter's columns, stack the ranks, drop the padding rows."""
    R = [-(-s[0] // W) for s in shapes]
    K = [int(np.prod(s[1:], dtype=np.int64)) for s in shapes]
    S = sum(r * k for r, k in zip(R, K))
    view = np.asarray(rank_major).reshape(W, S)
    out, col = [], 0
    for p, s in enumerate(shapes):
        n = R[p] * K[p]
        stacked = view[:, col:col + n].reshape(W * R[p], K[p])
        out.append(stacked[:s[0]].reshape(s))
        col += n
    return out


def check_copyout_worked_golden(orc):
    g = goldens.read("copyout_worked.txt")
    W = int(g["world"][0][0])
    shapes = [tuple(goldens.ints(s)) for s in g["shape"]]
    rm = goldens.hex16(g["rank_major"][0])
    got = orc.copyout(W, shapes, rm)
    for row in g["param"]:
        p = int(row[0])
        assert np.array_equal(got[p].reshape(-1), goldens.hex16(row[1:])), p


def check_copyout_round_trip(orc, seed=12):
    rng = np.random.default_rng(seed)
    cases = [(4, TINY_SHAPES), (1, [(3, 2), (5,)]), (8, [(6, 5120 // 512)])]
    for W in (2, 3, 4, 8):
        for _ in range(5):
            cases.append((W, random_case(rng, W, int(rng.integers(1, 6)))))
    for W, shapes in cases:
        X = [rng.integers(0, 0x10000, size=s, dtype=np.uint16) for s in shapes]
        rm = orc.pack(W, shapes, X)
        geo = orc.plan(W, shapes)
        assert rm.size == W * geo["S"]
        back = orc.copyout(W, shapes, rm)
        for p in range(len(shapes)):
            assert np.array_equal(back[p], X[p]), (W, shapes, p)


def check_copyout_matches_stock_and_skips_padding(orc, seed=13):
    rng = np.random.default_rng(seed)
    for W in (2, 4, 8):
        for _ in range(5):
            shapes = random_case(rng, W, int(rng.integers(1, 6)))
            geo = orc.plan(W, shapes)
            rm = rng.integers(0, 0x10000, size=W * geo["S"], dtype=np.uint16)
            got = orc.copyout(W, shapes, rm)
            want = stock_fsdp2_copyout(W, shapes, rm)
            for p in range(len(shapes)):
                assert np.array_equal(got[p], want[p])
            # padding slots changed to canaries: the copy-out result is the same
            X = [np.asarray(g).copy() for g in got]
            packed = orc.pack(W, shapes, X)
            canary = packed.copy()
            for p in range(len(shapes)):
                for r in range(W):
                    a = geo["rank_major_offset"][p, r]
                    canary[a + geo["n_real"][p, r]:a + geo["n"][p]] = 0x7FC1
                    assert np.all(packed[a + geo["n_real"][p, r]:a + geo["n"][p]] == 0)
            again = orc.copyout(W, shapes, canary)
            for p in range(len(shapes)):
                assert np.array_equal(again[p], X[p])


# --------------------------------------------------------------- copy-in


def check_cast_worked_golden(orc):
    g = goldens.read("cast_worked.txt")
    x = np.array([int(r[0], 16) for r in g["cast"]], dtype=np.uint32).view(np.float32)
    want = np.array([int(r[1], 16) for r in g["cast"]], dtype=np.uint16)
    got = orc.cast_bf16(x)
    bad = [(hex(int(a)), hex(int(b)), hex(int(c))) for a, b, c in zip(x.view(np.uint32), got, want) if b != c]
    assert not bad, bad


def check_cast_matches_torch_rne(orc, seed=14):
    """The cast equals torch's float32 -> bfloat16 conversion (round to nearest
    even) on every non-NaN input, and keeps NaNs NaN."""
    import torch

    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),
        rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    got = orc.cast_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)
    assert np.array_equal(got[nan] >> 15, (x[nan].view(np.uint32) >> 31).astype(np.uint16))


def shards_of(world, shapes, X):
    """Each rank's local shard of each parameter: its real rows, as views."""
    out = [[None] * len(shapes) for _ in range(world)]
    for p, s in enumerate(shapes):
        D = s[0]
        R = -(-D // world)
        rows = np.asarray(X[p]).reshape((D,) + tuple(s[1:]))
        for r in range(world):
            out[r][p] = rows[min(r * R, D):min((r + 1) * R, D)]
    return out


def check_copyin_bf16_equals_pack_and_round_trips(orc, seed=15):
    rng = np.random.default_rng(seed)
    for W in (1, 2, 3, 4, 8):
        shapes = random_case(rng, W, int(rng.integers(1, 6)))
        X = [rng.integers(0, 0x10000, size=s, dtype=np.uint16) for s in shapes]
        rm = orc.copyin(W, shapes, shards_of(W, shapes, X))
        assert np.array_equal(rm, orc.pack(W, shapes, X))
        back = orc.copyout(W, shapes, rm)
        for p in range(len(shapes)):
            assert np.array_equal(back[p], X[p])


def check_copyin_f32_is_cast_then_stock_pack(orc, seed=16):
    """fp32 shards: the result equals the stock path, i.e. torch's bf16 cast of
    the whole parameter followed by zero-padded rank-major packing."""
    import torch

    rng = np.random.default_rng(seed)
    for W in (2, 4, 8):
        shapes = random_case(rng, W, int(rng.integers(1, 6)))
        X = [(rng.standard_normal(s) * rng.choice([1e-3, 1.0, 1e30])).astype(np.float32) for s in shapes]
        rm = orc.copyin(W, shapes, shards_of(W, shapes, X))
        cast = [torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16) for x in X]
        R = [-(-s[0] // W) for s in shapes]
        K = [int(np.prod(s[1:], dtype=np.int64)) for s in shapes]
        want = []
        for r in range(W):
            for p, s in enumerate(shapes):
                padded = np.zeros((W * R[p], K[p]), dtype=np.uint16)
                padded[:s[0]] = cast[p].reshape(s[0], K[p])
                want.append(padded[r * R[p]:(r + 1) * R[p]].reshape(-1))
        want = np.concatenate(want) if want else np.zeros(0, np.uint16)
        assert np.array_equal(rm, want), (W, shapes)


# ------------------------------------------ Equation 5 in full, stock pack


def rand_f32(rng, shape, scale=1.0):
    return (rng.standard_normal(int(np.prod(shape, dtype=np.int64))) * scale).astype(np.float32).reshape(shape)


def check_rs_ex_defaults_are_the_base_case(orc, seed=17):
    rng = np.random.default_rng(seed)
    for W in (1, 3, 4, 8):
        shapes = random_case(rng, W, 4)
        grads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
        base = orc.rs_local(W, shapes, grads)
        ex = orc.rs_local_ex(W, shapes, grads)
        for r in range(W):
            assert same_bits(base[r], ex[r])


def check_rs_ex_fp32_grads(orc, seed=18):
    """fp32 gradients: the stock path's sum, and the bf16 path's result when
    every value is a bf16 value."""
    rng = np.random.default_rng(seed)
    for W in (2, 4, 8):
        shapes = random_case(rng, W, 4)
        grads = [[rand_f32(rng, s, scale=float(rng.choice([1e-3, 1.0, 1e3]))) for s in shapes] for _ in range(W)]
        got = orc.rs_local_ex(W, shapes, grads)
        want = stock_fsdp2_reduce_scatter(W, shapes, grads)
        for r in range(W):
            assert same_bits(got[r], want[r])
        bgrads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
        as_f32 = [[f32_from_bf16(g).reshape(g.shape) for g in row] for row in bgrads]
        a, b = orc.rs_local(W, shapes, bgrads), orc.rs_local_ex(W, shapes, as_f32)
        for r in range(W):
            assert same_bits(a[r], b[r])


def check_rs_ex_alpha(orc, seed=19):
    """alpha = 2^k scales exactly; alpha = -1 flips every sign (padding
    becomes -0); any alpha is one binary32 product of the sum."""
    rng = np.random.default_rng(seed)
    W = 4
    shapes = [(2 * W + 1, 5), (7,), (1, 3)]
    grads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
    base = orc.rs_local(W, shapes, grads)
    for k in (-3, 1, 5):
        got = orc.rs_local_ex(W, shapes, grads, alpha=2.0 ** k)
        for r in range(W):
            assert same_bits(got[r], base[r] * np.float32(2.0 ** k))
    neg = orc.rs_local_ex(W, shapes, grads, alpha=-1.0)
    for r in range(W):
        assert np.array_equal(neg[r].view(np.uint32), base[r].view(np.uint32) ^ np.uint32(0x80000000))
    tenth = orc.rs_local_ex(W, shapes, grads, alpha=0.1)
    for r in range(W):
        assert same_bits(tenth[r], np.float32(0.1) * base[r])


def check_rs_ex_accumulate(orc, seed=20):
    rng = np.random.default_rng(seed)
    for W in (2, 8):
        shapes = random_case(rng, W, 4)
        # integer values: the accumulated result is the exact integer sum
        ints = [[rng.integers(-64, 65, size=s) for s in shapes] for _ in range(W)]
        grads = [[(np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16) for v in row]
                 for row in ints]
        geo = orc.plan(W, shapes)
        old = [rng.integers(-1000, 1001, size=geo["S"]).astype(np.float32) for _ in range(W)]
        base = orc.rs_local(W, shapes, grads)
        got = orc.rs_local_ex(W, shapes, grads, alpha=1.0, accumulate=True, out=old)
        for r in range(W):
            assert np.array_equal(got[r].astype(np.int64), old[r].astype(np.int64) + base[r].astype(np.int64))
        # general values: one product, then one sum, each rounded
        fgrads = [[rand_bf16(rng, s) for s in shapes] for _ in range(W)]
        fold = [rand_f32(rng, (geo["S"],)) for _ in range(W)]
        fbase = orc.rs_local(W, shapes, fgrads)
        got = orc.rs_local_ex(W, shapes, fgrads, alpha=0.25, accumulate=True, out=fold)
        for r in range(W):
            assert same_bits(got[r], fold[r] + np.float32(0.25) * fbase[r])


def check_chunk_cat_matches_stock_pack(orc, seed=21):
    rng = np.random.default_rng(seed)
    for W in (1, 3, 4, 8):
        shapes = random_case(rng, W, int(rng.integers(1, 6)))
        g = [rand_bf16(rng, s) for s in shapes]
        got = orc.chunk_cat(W, shapes, g)
        want = stock_fsdp2_pack(W, shapes, g)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def check_eq5_worked_golden(orc):
    """Hand-worked Equation 5 cases: the product and the accumulation are two
    separate roundings, padding contributes +0 scaled by alpha."""
    g = goldens.read("eq5_worked.txt")
    cases = sorted({k.split(".")[0] for k in g})
    for c in cases:
        shape = (int(g[c + ".shape"][0][0]),)
        grads = [None, None]
        for row in g[c + ".grad"]:
            grads[int(row[0])] = [goldens.hex16(row[1:])]
        alpha = np.array([int(g[c + ".alpha"][0][0], 16)], dtype=np.uint32).view(np.float32)[0]
        acc = bool(int(g[c + ".accumulate"][0][0]))
        old = [None, None]
        want = [None, None]
        for row in g[c + ".old"]:
            old[int(row[0])] = np.array([int(v, 16) for v in row[1:]], dtype=np.uint32).view(np.float32)
        for row in g[c + ".out"]:
            want[int(row[0])] = np.array([int(v, 16) for v in row[1:]], dtype=np.uint32).view(np.float32)
        got = orc.rs_local_ex(2, [shape], grads, alpha, acc, old)
        for r in range(2):
            assert same_bits(got[r], want[r]), (c, r, got[r].view(np.uint32), want[r].view(np.uint32))


# ---------------------------------------------------- interference victim


def check_axpb_worked_golden(orc):
    g = goldens.read("axpb_worked.txt")
    cols = [np.array([int(r[i], 16) for r in g["axpb"]], dtype=np.uint32) for i in range(4)]
    x, a, b, want = cols
    for i in range(len(x)):
        got = orc.axpb(x[i:i + 1].view(np.float32), a[i:i + 1].view(np.float32)[0], b[i:i + 1].view(np.float32)[0])
        gb, wb = got.view(np.uint32)[0], want[i]
        if np.isnan(want[i:i + 1].view(np.float32)[0]):
            assert np.isnan(got[0]), (i, hex(gb))
        else:
            assert gb == wb, (i, hex(gb), hex(wb))


def check_axpb_integers_are_exact(orc, seed=22):
    """Small integers: every product and sum is exact, so the result is
    integer arithmetic's."""
    rng = np.random.default_rng(seed)
    xi = rng.integers(-2**10, 2**10, size=10000)
    for a, b in ((3, -7), (-1, 0), (0, 5), (1024, 1)):
        got = orc.axpb(xi.astype(np.float32), a, b)
        assert np.array_equal(got, (a * xi + b).astype(np.float32)), (a, b)


def check_axpb_is_two_numpy_float32_operations(orc, seed=23):
    """numpy's float32 multiply then float32 add (each one IEEE rounding) give
    the same bits on random and special inputs."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([(rng.standard_normal(100000) * 10.0 ** rng.integers(-44, 37, 100000)).astype(np.float32),
                        np.array([0x00000001, 0x807FFFFF, 0x7F7FFFFF], dtype=np.uint32).view(np.float32)])
    for a, b in ((np.float32(0.1), np.float32(0.7)), (np.float32(-3.0e38), np.float32(1e-30)),
                 (np.float32(1.0 + 2 ** -12), np.float32(-1.0))):
        with np.errstate(all="ignore"):
            want = (x * a) + b
        got = orc.axpb(x, a, b)
        assert same_bits(got, want), (a, b)


ALL_CHECKS = [
    check_tiny_plan_golden,
    check_plan_invariants,
    check_landing_is_padded_parameter,
    check_rs_worked_golden,
    check_rs_matches_stock_path,
    check_rs_w1_identity,
    check_rs_integer_inputs_exact,
    check_rs_identical_ranks,
    check_rs_one_hot_rank,
    check_rs_sum_over_ranks,
    check_rs_fp64_bounds,
    check_rs_thread_invariance,
    check_rs_special_values,
    check_rs_padding_positive_zero,
    check_rs_linearity,
    check_copyout_worked_golden,
    check_copyout_round_trip,
    check_copyout_matches_stock_and_skips_padding,
    check_cast_worked_golden,
    check_cast_matches_torch_rne,
    check_copyin_bf16_equals_pack_and_round_trips,
    check_copyin_f32_is_cast_then_stock_pack,
    check_rs_ex_defaults_are_the_base_case,
    check_rs_ex_fp32_grads,
    check_rs_ex_alpha,
    check_rs_ex_accumulate,
    check_chunk_cat_matches_stock_pack,
    check_eq5_worked_golden,
    check_axpb_worked_golden,
    check_axpb_integers_are_exact,
    check_axpb_is_two_numpy_float32_operations,
]
