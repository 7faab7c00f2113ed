"""CPU oracle for the RS-local reduce and the AG copy-out (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares no code with the HIP library.  The arithmetic lives in
``tide_oracle.c`` (plain C loops); this module only marshals numpy arrays.

Definitions followed ("The Endgame of FSDP Communication: Layout-Aware
Collectives on Copy Engines, RDMA, and NVSwitch", Wang et al.):
  * ``plan``     -- Section 2.1, shard geometry and Equation 2 (landing offset);
  * ``rs_local`` -- Section 4, Equation 5 (alpha = 1, accumulate = 0), summed
                    in rank order 0..W-1 in binary32 (Section 4.3);
  * ``copyout``  -- Section 2.1, rank-major all-gather output to per-parameter
                    storage;
  * ``pack``     -- Section 2.1, the inverse (FSDP2's copy-in), padding zero;
  * ``rs_local_ex`` -- Section 4, Equation 5 in full: alpha, accumulate,
                    bf16 or fp32 gradients;
  * ``chunk_cat`` -- Section 2.1, Equation 3: stock FSDP2's packed fp32
                    reduce-scatter input of one rank (the baseline);
  * ``copyin``   -- Sections 2.1 and 3.1: every rank's local shards (fp32 cast
                    to bf16 by round to nearest even, or bf16 as is) into the
                    rank-major buffer, padding zero.

bf16 values are carried as ``numpy.uint16`` bit patterns throughout.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtide_oracle.so")


class OracleError(RuntimeError):
    pass


def _bind(lib):
    i32, i64p, i32p = ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.oracle_plan.argtypes = [i32, i32, i32p, i64p] + [i64p] * 9
    lib.oracle_plan.restype = ctypes.c_int
    lib.oracle_rs_local.argtypes = [i32, i32, i32p, i64p, vpp, vpp, i32]
    lib.oracle_rs_local.restype = ctypes.c_int
    lib.oracle_copyout.argtypes = [i32, i32, i32p, i64p, ctypes.c_void_p, vpp, i32]
    lib.oracle_copyout.restype = ctypes.c_int
    lib.oracle_pack.argtypes = [i32, i32, i32p, i64p, vpp, ctypes.c_void_p, i32]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_copyin.argtypes = [i32, i32, i32p, i64p, vpp, i32, ctypes.c_void_p, i32]
    lib.oracle_copyin.restype = ctypes.c_int
    lib.oracle_cast_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_cast_bf16.restype = ctypes.c_int
    lib.oracle_rs_local_ex.argtypes = [i32, i32, i32p, i64p, vpp, i32, ctypes.c_float, i32, vpp, i32]
    lib.oracle_rs_local_ex.restype = ctypes.c_int
    lib.oracle_chunk_cat.argtypes = [i32, i32, i32p, i64p, vpp, ctypes.c_void_p, i32]
    lib.oracle_chunk_cat.restype = ctypes.c_int
    lib.oracle_axpb.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    lib.oracle_axpb.restype = ctypes.c_int
    return lib


def _shape_args(shapes):
    ndims = np.array([len(s) for s in shapes], dtype=np.int32)
    dims = np.array([d for s in shapes for d in s] or [0], dtype=np.int64)
    return ndims, dims


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _ptrs(arrays):
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def _as_u16(a, n, what):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{what}: expected uint16 bf16 bit patterns, got {a.dtype}")
    if a.size != n:
        raise ValueError(f"{what}: expected {n} elements, got {a.size}")
    return a.reshape(-1)


class Oracle:
    """The oracle functions, bound to one build of ``tide_oracle.c``."""

    def __init__(self, lib_path=_LIB_PATH):
        if not os.path.exists(lib_path):
            if lib_path != _LIB_PATH:
                raise FileNotFoundError(lib_path)
            from oracle.build import build_oracle

            build_oracle()
        self.lib = _bind(ctypes.CDLL(lib_path))

    def plan(self, world, shapes):
        """Shard geometry: dict of numpy arrays D, K, R, n, o ([P]), S (int), and
        n_real, rank_major_offset, landing_offset ([P, W])."""
        P = len(shapes)
        ndims, dims = _shape_args(shapes)
        out = {k: np.zeros(P, dtype=np.int64) for k in ("D", "K", "R", "n", "o")}
        S = np.zeros(1, dtype=np.int64)
        per = {k: np.zeros((P, world), dtype=np.int64) for k in ("n_real", "rank_major_offset", "landing_offset")}
        rc = self.lib.oracle_plan(world, P, _i32p(ndims), _i64p(dims), _i64p(out["D"]), _i64p(out["K"]),
                                  _i64p(out["R"]), _i64p(out["n"]), _i64p(out["o"]), _i64p(S),
                                  _i64p(per["n_real"]), _i64p(per["rank_major_offset"]),
                                  _i64p(per["landing_offset"]))
        _check(rc, "oracle_plan")
        out.update(per)
        out["S"] = int(S[0])
        return out

    def rs_local(self, world, shapes, grads, nthreads=1):
        """grads[u][p]: rank u's bf16 gradient of parameter p (uint16 bits,
        D_p*K_p elements).  Returns the W packed fp32 shards (float32, S each)."""
        geo = self.plan(world, shapes)
        P = len(shapes)
        if len(grads) != world or any(len(g) != P for g in grads):
            raise ValueError("grads must be indexed [rank][parameter]")
        flat = []
        for u in range(world):
            for p in range(P):
                flat.append(_as_u16(grads[u][p], int(geo["D"][p] * geo["K"][p]), f"grads[{u}][{p}]"))
        outs = [np.empty(max(geo["S"], 1), dtype=np.float32) for _ in range(world)]
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_rs_local(world, P, _i32p(ndims), _i64p(dims), _ptrs(flat), _ptrs(outs), int(nthreads))
        _check(rc, "oracle_rs_local")
        return [o[: geo["S"]] for o in outs]

    def copyout(self, world, shapes, rank_major, nthreads=1):
        """rank_major: W*S bf16 bits.  Returns the P parameters (uint16, shaped)."""
        geo = self.plan(world, shapes)
        rm = _as_u16(rank_major, world * geo["S"], "rank_major")
        if rm.size == 0:
            rm = np.zeros(1, dtype=np.uint16)
        params = [np.empty(max(int(geo["D"][p] * geo["K"][p]), 1), dtype=np.uint16) for p in range(len(shapes))]
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_copyout(world, len(shapes), _i32p(ndims), _i64p(dims), rm.ctypes.data,
                                     _ptrs(params), int(nthreads))
        _check(rc, "oracle_copyout")
        return [params[p][: int(geo["D"][p] * geo["K"][p])].reshape(shapes[p]) for p in range(len(shapes))]

    def pack(self, world, shapes, params, nthreads=1):
        """params[p]: D_p*K_p bf16 bits.  Returns the rank-major buffer (W*S uint16)."""
        geo = self.plan(world, shapes)
        flat = []
        for p in range(len(shapes)):
            a = _as_u16(params[p], int(geo["D"][p] * geo["K"][p]), f"params[{p}]")
            flat.append(a if a.size else np.zeros(1, dtype=np.uint16))
        rm = np.empty(max(world * geo["S"], 1), dtype=np.uint16)
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_pack(world, len(shapes), _i32p(ndims), _i64p(dims), _ptrs(flat), rm.ctypes.data,
                                  int(nthreads))
        _check(rc, "oracle_pack")
        return rm[: world * geo["S"]]


    def copyin(self, world, shapes, shards, nthreads=1):
        """shards[r][p]: rank r's local shard of parameter p, n_real(p, r)
        elements, all float32 (cast) or all uint16 bf16 bits (copied).
        Returns the rank-major buffer (W*S uint16)."""
        geo = self.plan(world, shapes)
        P = len(shapes)
        if len(shards) != world or any(len(s) != P for s in shards):
            raise ValueError("shards must be indexed [rank][parameter]")
        dtypes = {np.asarray(a).dtype for row in shards for a in row}
        if dtypes not in ({np.dtype(np.float32)}, {np.dtype(np.uint16)}):
            raise TypeError(f"shards must be all float32 or all uint16, got {dtypes}")
        f32 = dtypes == {np.dtype(np.float32)}
        flat = []
        for r in range(world):
            for p in range(P):
                a = np.ascontiguousarray(shards[r][p]).reshape(-1)
                if a.size != geo["n_real"][p, r]:
                    raise ValueError(f"shards[{r}][{p}]: expected {geo['n_real'][p, r]} elements, got {a.size}")
                flat.append(a if a.size else np.zeros(1, dtype=a.dtype))
        rm = np.empty(max(world * geo["S"], 1), dtype=np.uint16)
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_copyin(world, P, _i32p(ndims), _i64p(dims), _ptrs(flat), 1 if f32 else 0,
                                    rm.ctypes.data, int(nthreads))
        _check(rc, "oracle_copyin")
        return rm[: world * geo["S"]]

    def rs_local_ex(self, world, shapes, grads, alpha=1.0, accumulate=False, out=None, nthreads=1):
        """Equation 5 in full: grads[u][p] all uint16 (bf16 bits) or all
        float32; out (W float32 arrays of S, read when accumulating) is
        updated in place and returned (new arrays when None)."""
        geo = self.plan(world, shapes)
        P = len(shapes)
        if len(grads) != world or any(len(g) != P for g in grads):
            raise ValueError("grads must be indexed [rank][parameter]")
        dtypes = {np.asarray(a).dtype for row in grads for a in row}
        if dtypes not in ({np.dtype(np.float32)}, {np.dtype(np.uint16)}):
            raise TypeError(f"grads must be all float32 or all uint16, got {dtypes}")
        f32 = dtypes == {np.dtype(np.float32)}
        flat = []
        for u in range(world):
            for p in range(P):
                a = np.ascontiguousarray(grads[u][p]).reshape(-1)
                if a.size != geo["D"][p] * geo["K"][p]:
                    raise ValueError(f"grads[{u}][{p}] has {a.size} elements")
                flat.append(a if a.size else np.zeros(1, dtype=a.dtype))
        if out is None:
            out = [np.zeros(max(geo["S"], 1), dtype=np.float32) for _ in range(world)]
        else:
            out = [np.ascontiguousarray(o, dtype=np.float32).copy() if o.size else np.zeros(1, np.float32)
                   for o in out]
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_rs_local_ex(world, P, _i32p(ndims), _i64p(dims), _ptrs(flat), 1 if f32 else 0,
                                         float(alpha), int(bool(accumulate)), _ptrs(out), int(nthreads))
        _check(rc, "oracle_rs_local_ex")
        return [o[: geo["S"]] for o in out]

    def chunk_cat(self, world, shapes, grads_u, nthreads=1):
        """Stock FSDP2 packing of one rank's bf16 gradients grads_u[p] ->
        float32 array of W*S."""
        geo = self.plan(world, shapes)
        flat = []
        for p in range(len(shapes)):
            a = _as_u16(grads_u[p], int(geo["D"][p] * geo["K"][p]), f"grads_u[{p}]")
            flat.append(a if a.size else np.zeros(1, dtype=np.uint16))
        packed = np.empty(max(world * geo["S"], 1), dtype=np.float32)
        ndims, dims = _shape_args(shapes)
        rc = self.lib.oracle_chunk_cat(world, len(shapes), _i32p(ndims), _i64p(dims), _ptrs(flat),
                                       packed.ctypes.data, int(nthreads))
        _check(rc, "oracle_chunk_cat")
        return packed[: world * geo["S"]]

    def cast_bf16(self, x):
        """float32 array -> bf16 bits (uint16), the copy-in's cast."""
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        out = np.empty(max(x.size, 1), dtype=np.uint16)
        _check(self.lib.oracle_cast_bf16(x.ctypes.data, x.size, out.ctypes.data), "oracle_cast_bf16")
        return out[: x.size]


    def axpb(self, x, a, b):
        """The elementwise victim: float32 y = a * x + b, two roundings."""
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        y = np.empty(max(x.size, 1), dtype=np.float32)
        _check(self.lib.oracle_axpb(x.size, x.ctypes.data, float(a), float(b), y.ctypes.data), "oracle_axpb")
        return y[: x.size]


_default = None


def _get():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def plan(world, shapes):
    return _get().plan(world, shapes)


def rs_local(world, shapes, grads, nthreads=1):
    return _get().rs_local(world, shapes, grads, nthreads)


def copyout(world, shapes, rank_major, nthreads=1):
    return _get().copyout(world, shapes, rank_major, nthreads)


def pack(world, shapes, params, nthreads=1):
    return _get().pack(world, shapes, params, nthreads)


def copyin(world, shapes, shards, nthreads=1):
    return _get().copyin(world, shapes, shards, nthreads)


def cast_bf16(x):
    return _get().cast_bf16(x)


def rs_local_ex(world, shapes, grads, alpha=1.0, accumulate=False, out=None, nthreads=1):
    return _get().rs_local_ex(world, shapes, grads, alpha, accumulate, out, nthreads)


def chunk_cat(world, shapes, grads_u, nthreads=1):
    return _get().chunk_cat(world, shapes, grads_u, nthreads)


def axpb(x, a, b):
    return _get().axpb(x, a, b)
