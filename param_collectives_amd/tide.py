"""Python binding of libtide (include/tide.h): argument marshalling only.

Every step of the reduce-scatter local stage, the all-gather copy-out and
copy-in, and the stock gradient pack runs in the HIP library; this module turns torch tensors into device pointers and
the current HIP stream, checks that each tensor has the size, dtype, device
and contiguity the plan expects (so that no kernel is launched on a buffer
smaller than the plan assumes), and raises on a non-zero status.  There is no
fallback: without the compiled library, importing this module fails.
"""
import ctypes
import os

import numpy as np

# PyTorch ships its own HIP runtime under the same soname as the system's, and
# whichever copy a process loads first serves every library in it.  torch is
# imported before the library is loaded, so that torch and this library share
# one runtime (its devices, memory and streams).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libtide.so")

TIDE_OK = 0
STATUS_NAMES = {
    0: "TIDE_OK",
    -1: "TIDE_ERR_INVALID",
    -2: "TIDE_ERR_RANGE",
    -3: "TIDE_ERR_ALIGN",
    -4: "TIDE_ERR_NOMEM",
    -5: "TIDE_ERR_HIP",
    -6: "TIDE_ERR_UNSUPPORTED",
}
FLAG_CACHED_LOADS = 0x1
FLAG_CACHED_STORES = 0x2
FLAG_NO_LDS = 0x4
DTYPE_BF16 = 0
DTYPE_F32 = 1
MAX_WORLD = 256
NOALLOC_SCRATCH_BYTES = 1 << 20

# Every symbol include/tide.h declares.
EXPORTS = (
    "tide_plan_create",
    "tide_plan_layout",
    "tide_plan_sizes",
    "tide_plan_segments",
    "tide_plan_set_options",
    "tide_plan_get_options",
    "tide_plan_launches",
    "tide_plan_paths",
    "tide_reduce_scatter_local",
    "tide_reduce_scatter_local_noalloc",
    "tide_allgather_copyout",
    "tide_allgather_copyin",
    "tide_reduce_scatter_local_f32",
    "tide_stock_chunk_cat",
    "tide_device_info",
    "tide_probe_launch",
    "tide_victim_axpb",
    "tide_stream_create",
    "tide_stream_destroy",
    "tide_plan_destroy",
    "tide_last_error",
)


class TideError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Options(ctypes.Structure):
    _fields_ = [("cu_budget", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32),
                ("chunk_elems", ctypes.c_int64), ("flags", ctypes.c_uint32), ("wave_chunks", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing: build it with `python param_collectives_amd/build.py` "
                          "(the HIP path has no fallback)")
    lib = ctypes.CDLL(LIBRARY)
    vp, i32, i64, i64p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)
    lib.tide_plan_create.argtypes = [i32, i32, ctypes.POINTER(i32), i64p, ctypes.POINTER(Options),
                                     ctypes.POINTER(vp)]
    lib.tide_plan_layout.argtypes = [vp, i64p, i64p, i64p]
    lib.tide_plan_sizes.argtypes = [vp, i64p, i64p]
    lib.tide_plan_segments.argtypes = [vp, i32, i64p, i64, i64p]
    lib.tide_plan_set_options.argtypes = [vp, ctypes.POINTER(Options)]
    lib.tide_plan_get_options.argtypes = [vp, i32, ctypes.POINTER(Options)]
    lib.tide_plan_launches.argtypes = [vp, i32, i32, i64p, i64, i64p]
    lib.tide_plan_paths.argtypes = [vp, i32, i64p]
    lib.tide_reduce_scatter_local.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_float, i32, vp]
    lib.tide_allgather_copyout.argtypes = [vp, vp, ctypes.POINTER(vp), vp]
    lib.tide_allgather_copyin.argtypes = [vp, ctypes.POINTER(vp), i32, vp, vp]
    lib.tide_reduce_scatter_local_f32.argtypes = lib.tide_reduce_scatter_local.argtypes
    lib.tide_reduce_scatter_local_noalloc.argtypes = lib.tide_reduce_scatter_local.argtypes
    lib.tide_stock_chunk_cat.argtypes = [vp, ctypes.POINTER(vp), vp, vp]
    i32p = ctypes.POINTER(i32)
    lib.tide_device_info.argtypes = [i32p, i32p, i32p, i32p]
    lib.tide_probe_launch.argtypes = [vp, i32, i32, i64, vp]
    lib.tide_victim_axpb.argtypes = [vp, vp, i64, ctypes.c_float, ctypes.c_float, vp]
    lib.tide_stream_create.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32, ctypes.POINTER(vp)]
    lib.tide_stream_destroy.argtypes = [vp]
    lib.tide_plan_destroy.argtypes = [vp]
    lib.tide_plan_destroy.restype = None
    lib.tide_last_error.argtypes = []
    lib.tide_last_error.restype = ctypes.c_char_p
    for name in EXPORTS[:-2]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _check(status):
    if status != TIDE_OK:
        raise TideError(status, lib.tide_last_error().decode(errors="replace"))


def _options(cu_budget=0, wg_per_cu=0, chunk_elems=0, flags=0, wave_chunks=0):
    return Options(int(cu_budget), int(wg_per_cu), int(chunk_elems), int(flags), int(wave_chunks))


def _ptr_array(values):
    return (ctypes.c_void_p * max(len(values), 1))(*[int(v) if v else None for v in values])


class Plan:
    """A shard-layout plan for `world` simulated ranks and the given parameter
    shapes (tide_plan_create)."""

    def __init__(self, world, shapes, cu_budget=0, wg_per_cu=0, chunk_elems=0, flags=0, wave_chunks=0):
        self.world = int(world)
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        ndims = (ctypes.c_int32 * max(len(self.shapes), 1))(*[len(s) for s in self.shapes])
        flat = [d for s in self.shapes for d in s]
        dims = (ctypes.c_int64 * max(len(flat), 1))(*flat)
        handle = ctypes.c_void_p()
        opt = _options(cu_budget, wg_per_cu, chunk_elems, flags, wave_chunks)
        _check(lib.tide_plan_create(self.world, len(self.shapes), ndims, dims, ctypes.byref(opt),
                                    ctypes.byref(handle)))
        self.handle = handle
        R = np.zeros(len(self.shapes), dtype=np.int64)
        o = np.zeros(len(self.shapes), dtype=np.int64)
        S = np.zeros(1, dtype=np.int64)
        _check(lib.tide_plan_layout(self.handle, R.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    o.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    S.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        self.rows_per_rank, self.shard_offset, self.shard_elems = R, o, int(S[0])
        # element counts as the library sizes them: numel[p] of parameter p,
        # n_real[r][p] of rank r's shard of p (its real, non-padding elements)
        numel = np.zeros(len(self.shapes), dtype=np.int64)
        real = np.zeros(self.world * len(self.shapes), dtype=np.int64)
        _check(lib.tide_plan_sizes(self.handle, numel.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   real.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        self.numel = [int(v) for v in numel]
        self.n_real = real.reshape(self.world, len(self.shapes)).tolist()

    def segments(self, op):
        """The work segments (op 0: reduce-scatter, 1: copy-out, 2: copy-in,
        3: stock pack, 4: reduce-scatter of fp32 gradients) as an int64 array
        of rows (kind, src_idx, dst_idx, src_off, dst_off, len)."""
        count = ctypes.c_int64()
        _check(lib.tide_plan_segments(self.handle, int(op), None, 0, ctypes.byref(count)))
        table = np.zeros((max(count.value, 1), 6), dtype=np.int64)
        _check(lib.tide_plan_segments(self.handle, int(op), table.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      count.value, ctypes.byref(count)))
        return table[:count.value]

    def launches(self, op=0, cu_count=0):
        """The kernel launches one call of `op` makes under the current
        options, as an int64 array of rows (first chunk, end chunk, first
        segment, end segment, workgroups); cu_count stands for a cu_budget of
        0 (0: the bound device's CU count)."""
        count = ctypes.c_int64()
        _check(lib.tide_plan_launches(self.handle, int(op), int(cu_count), None, 0, ctypes.byref(count)))
        table = np.zeros((max(count.value, 1), 5), dtype=np.int64)
        _check(lib.tide_plan_launches(self.handle, int(op), int(cu_count),
                                      table.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), count.value,
                                      ctypes.byref(count)))
        return table[:count.value]

    def paths(self, op=0):
        """Elements of the latest call of `op` by code path (tide_plan_paths):
        dict of vector, realigned and element-by-element counts, and whether a
        reduce-scatter ran its realigning instance."""
        out = np.zeros(4, dtype=np.int64)
        _check(lib.tide_plan_paths(self.handle, int(op), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return {"vector": int(out[0]), "realigned": int(out[1]), "element": int(out[2]),
                "realigning_instance": bool(out[3])}

    def set_options(self, cu_budget=0, wg_per_cu=0, chunk_elems=0, flags=0, wave_chunks=0):
        opt = _options(cu_budget, wg_per_cu, chunk_elems, flags, wave_chunks)
        _check(lib.tide_plan_set_options(self.handle, ctypes.byref(opt)))

    def options(self, op=0):
        """Effective launch knobs for op 0 (reduce-scatter), 1 (copy-out),
        2 (copy-in), 3 (stock pack) or 4 (reduce-scatter of fp32 gradients)."""
        opt = Options()
        _check(lib.tide_plan_get_options(self.handle, int(op), ctypes.byref(opt)))
        return {"cu_budget": opt.cu_budget, "wg_per_cu": opt.wg_per_cu, "chunk_elems": opt.chunk_elems,
                "flags": opt.flags, "wave_chunks": opt.wave_chunks}

    def destroy(self):
        if getattr(self, "handle", None):
            lib.tide_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    # ------------------------------------------------------------ raw calls

    @staticmethod
    def _lengths(values, n, what):
        # the library reads exactly n entries of each pointer array
        if len(values) != n:
            raise ValueError(f"{what} must hold {n} addresses, got {len(values)}")

    def reduce_scatter_local_raw(self, grad_ptrs, out_ptrs, alpha=1.0, accumulate=0, stream=0, f32=False):
        """tide_reduce_scatter_local (bf16 gradients) or, with f32=True,
        tide_reduce_scatter_local_f32 on raw device addresses: grad_ptrs[u*P+p],
        out_ptrs[r] (ints), stream a hipStream_t handle (int)."""
        self._lengths(grad_ptrs, self.world * len(self.shapes), "grad_ptrs")
        self._lengths(out_ptrs, self.world, "out_ptrs")
        fn = lib.tide_reduce_scatter_local_f32 if f32 else lib.tide_reduce_scatter_local
        _check(fn(self.handle, _ptr_array(grad_ptrs), _ptr_array(out_ptrs), float(alpha), int(accumulate),
                  ctypes.c_void_p(int(stream) or None)))

    def stock_chunk_cat_raw(self, grad_ptrs, packed_ptr, stream=0):
        """tide_stock_chunk_cat on raw device addresses (grad_ptrs[p] of one
        rank, packed_ptr to W*S fp32 elements)."""
        self._lengths(grad_ptrs, len(self.shapes), "grad_ptrs")
        _check(lib.tide_stock_chunk_cat(self.handle, _ptr_array(grad_ptrs), ctypes.c_void_p(int(packed_ptr) or None),
                                        ctypes.c_void_p(int(stream) or None)))

    def allgather_copyin_raw(self, shard_ptrs, shard_dtype, rank_major_ptr, stream=0):
        """tide_allgather_copyin on raw device addresses (shard_ptrs[r*P+p])."""
        self._lengths(shard_ptrs, self.world * len(self.shapes), "shard_ptrs")
        _check(lib.tide_allgather_copyin(self.handle, _ptr_array(shard_ptrs), int(shard_dtype),
                                         ctypes.c_void_p(int(rank_major_ptr) or None),
                                         ctypes.c_void_p(int(stream) or None)))

    def allgather_copyout_raw(self, rank_major_ptr, param_ptrs, stream=0):
        """tide_allgather_copyout on raw device addresses."""
        self._lengths(param_ptrs, len(self.shapes), "param_ptrs")
        _check(lib.tide_allgather_copyout(self.handle, ctypes.c_void_p(int(rank_major_ptr) or None),
                                          _ptr_array(param_ptrs), ctypes.c_void_p(int(stream) or None)))


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _require(t, dtype, numel, what):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: expected a GPU tensor, got {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what}: lives on {t.device}, but the kernels run on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if t.numel() != numel:
        raise ValueError(f"{what}: expected {numel} elements, got {t.numel()}")


class Call:
    """One operation with its tensors checked and its pointer arrays
    marshalled once (the buffers an FSDP2 group reuses every step); calling it
    launches on the given (or current) stream with a single library call.
    It holds references to the tensors, so they outlive it."""

    def __init__(self, fn, args, tensors):
        self._fn = fn
        self._args = args
        self._tensors = tensors

    def __call__(self, stream=None):
        _check(self._fn(*self._args, ctypes.c_void_p(_stream_handle(stream) or None)))


def _rs_checked(plan, grads, outs):
    """Checks the tensors of a reduce-scatter; returns (gradient pointers,
    output pointers, whether the gradients are fp32)."""
    import torch

    W, P = plan.world, len(plan.shapes)
    if len(grads) != W or any(len(row) != P for row in grads):
        raise ValueError(f"grads must be {W} lists of {P} tensors")
    if len(outs) != W:
        raise ValueError(f"outs must hold {W} tensors")
    dtypes = {t.dtype for row in grads for t in row}
    if dtypes not in ({torch.float32}, {torch.bfloat16}):
        raise TypeError(f"grads must be all torch.bfloat16 or all torch.float32, got {dtypes}")
    dtype = dtypes.pop()
    ptrs = []
    for u in range(W):
        for p in range(P):
            _require(grads[u][p], dtype, plan.numel[p], f"grads[{u}][{p}]")
            ptrs.append(grads[u][p].data_ptr())
    for r in range(W):
        _require(outs[r], torch.float32, plan.shard_elems, f"outs[{r}]")
    return ptrs, [o.data_ptr() for o in outs], dtype == torch.float32


def reduce_scatter_call(plan, grads, outs, alpha=1.0, accumulate=False):
    """A registered reduce-scatter (see reduce_scatter_local)."""
    g, o, f32 = _rs_checked(plan, grads, outs)
    fn = lib.tide_reduce_scatter_local_f32 if f32 else lib.tide_reduce_scatter_local
    return Call(fn, (plan.handle, _ptr_array(g), _ptr_array(o), ctypes.c_float(alpha), int(bool(accumulate))),
                (plan, grads, outs))


def reduce_scatter_local(plan, grads, outs, alpha=1.0, accumulate=False, stream=None):
    """Reduce-scatter local stage: grads[u][p] (all bf16 or all fp32,
    plan.shapes[p]) for u in [0, W) -> outs[r] (fp32, plan.shard_elems
    elements) for r in [0, W): outs[r] = alpha * (sum over u in rank order),
    added to the old outs[r] when accumulate is true."""
    g, o, f32 = _rs_checked(plan, grads, outs)
    plan.reduce_scatter_local_raw(g, o, alpha, int(bool(accumulate)), _stream_handle(stream), f32=f32)


def reduce_scatter_local_noalloc(plan, grads, outs, alpha=1.0, accumulate=False, stream=None):
    """The allocation-free reduce-scatter (tide_reduce_scatter_local_noalloc):
    the results of reduce_scatter_local from bf16 gradients, with the call's
    tables written to the library's fixed device scratch array instead of
    plan-owned device memory.  Calls that may overlap on one device race for
    that array."""
    g, o, f32 = _rs_checked(plan, grads, outs)
    if f32:
        raise TypeError("the allocation-free reduce-scatter takes bf16 gradients")
    _check(lib.tide_reduce_scatter_local_noalloc(plan.handle, _ptr_array(g), _ptr_array(o), ctypes.c_float(alpha),
                                                 int(bool(accumulate)),
                                                 ctypes.c_void_p(_stream_handle(stream) or None)))


def _pk_checked(plan, grads, packed):
    import torch

    P = len(plan.shapes)
    if len(grads) != P:
        raise ValueError(f"grads must hold {P} tensors (one rank's gradients)")
    for p in range(P):
        _require(grads[p], torch.bfloat16, plan.numel[p], f"grads[{p}]")
    _require(packed, torch.float32, plan.world * plan.shard_elems, "packed")
    return [t.data_ptr() for t in grads], packed.data_ptr()


def stock_chunk_cat_call(plan, grads, packed):
    """A registered stock gradient pack (see stock_chunk_cat)."""
    g, pk = _pk_checked(plan, grads, packed)
    return Call(lib.tide_stock_chunk_cat, (plan.handle, _ptr_array(g), ctypes.c_void_p(pk or None)),
                (plan, grads, packed))


def stock_chunk_cat(plan, grads, packed, stream=None):
    """Stock gradient pack of one rank: grads[p] (bf16, plan.shapes[p]) ->
    packed (fp32, W*S elements: rank r's rows of p at r*S + o_p, widened,
    padding +0)."""
    g, pk = _pk_checked(plan, grads, packed)
    plan.stock_chunk_cat_raw(g, pk, _stream_handle(stream))


def _co_checked(plan, rank_major, params):
    import torch

    P = len(plan.shapes)
    _require(rank_major, torch.bfloat16, plan.world * plan.shard_elems, "rank_major")
    if len(params) != P:
        raise ValueError(f"params must hold {P} tensors")
    for p in range(P):
        _require(params[p], torch.bfloat16, plan.numel[p], f"params[{p}]")
    return rank_major.data_ptr(), [t.data_ptr() for t in params]


def allgather_copyout_call(plan, rank_major, params):
    """A registered copy-out (see allgather_copyout)."""
    rm, ps = _co_checked(plan, rank_major, params)
    return Call(lib.tide_allgather_copyout, (plan.handle, ctypes.c_void_p(rm or None), _ptr_array(ps)),
                (plan, rank_major, params))


def allgather_copyout(plan, rank_major, params, stream=None):
    """All-gather copy-out: rank_major (bf16, W*S elements) -> params[p]
    (bf16, plan.shapes[p])."""
    rm, ps = _co_checked(plan, rank_major, params)
    plan.allgather_copyout_raw(rm, ps, _stream_handle(stream))


def _ci_checked(plan, shards, rank_major):
    import torch

    W, P = plan.world, len(plan.shapes)
    if len(shards) != W or any(len(row) != P for row in shards):
        raise ValueError(f"shards must be {W} lists of {P} tensors")
    dtypes = {t.dtype for row in shards for t in row}
    if dtypes not in ({torch.float32}, {torch.bfloat16}):
        raise TypeError(f"shards must be all torch.float32 or all torch.bfloat16, got {dtypes}")
    dtype = dtypes.pop()
    ptrs = []
    for r in range(W):
        for p in range(P):
            _require(shards[r][p], dtype, plan.n_real[r][p], f"shards[{r}][{p}]")
            ptrs.append(shards[r][p].data_ptr())
    _require(rank_major, torch.bfloat16, W * plan.shard_elems, "rank_major")
    return ptrs, DTYPE_F32 if dtype == torch.float32 else DTYPE_BF16, rank_major.data_ptr()


def allgather_copyin_call(plan, shards, rank_major):
    """A registered copy-in (see allgather_copyin)."""
    ptrs, dt, rm = _ci_checked(plan, shards, rank_major)
    return Call(lib.tide_allgather_copyin, (plan.handle, _ptr_array(ptrs), dt, ctypes.c_void_p(rm or None)),
                (plan, shards, rank_major))


def allgather_copyin(plan, shards, rank_major, stream=None):
    """All-gather copy-in: shards[r][p] (rank r's local shard of parameter p,
    n_real(p, r) elements, all float32 or all bfloat16) -> rank_major (bf16,
    W*S elements; fp32 shards are cast by round to nearest even)."""
    ptrs, dt, rm = _ci_checked(plan, shards, rank_major)
    plan.allgather_copyin_raw(ptrs, dt, rm, _stream_handle(stream))


# ------------------------------------------------------------ instruments


def device_info():
    """CU count, largest LDS allocation per workgroup and LDS per CU (bytes),
    and wall-clock rate (kHz) of the current device (tide_device_info)."""
    cu, lds, lds_cu, khz = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.tide_device_info(ctypes.byref(cu), ctypes.byref(lds), ctypes.byref(lds_cu), ctypes.byref(khz)))
    return {"cu_count": cu.value, "max_lds_per_workgroup": lds.value, "lds_per_cu": lds_cu.value,
            "wall_clock_khz": khz.value}


PROBE_WORDS = 8


def probe(records, grid, lds_bytes, hold_ns, stream=None):
    """Launch the hardware-ID probe (tide_probe_launch): `records` is a GPU
    int32 tensor of at least grid*8 elements; decode it with decode_probe."""
    import torch

    if not isinstance(records, torch.Tensor) or records.device.type != "cuda" or records.dtype != torch.int32:
        raise TypeError("records: expected a GPU torch.int32 tensor")
    if not records.is_contiguous() or records.numel() < int(grid) * PROBE_WORDS:
        raise ValueError(f"records: expected a contiguous tensor of at least {int(grid) * PROBE_WORDS} elements")
    _check(lib.tide_probe_launch(ctypes.c_void_p(records.data_ptr()), int(grid), int(lds_bytes), int(hold_ns),
                                 ctypes.c_void_p(_stream_handle(stream) or None)))


def decode_probe(records):
    """Probe records (any int32/uint32 array of grid*8 words) -> dict of numpy
    arrays: block, wave, simd, cu, sh, se, xcc, ok (LDS read back intact),
    entry, exit (wall-clock ticks)."""
    r = np.asarray(records).reshape(-1, PROBE_WORDS).view(np.uint32).astype(np.int64)
    hw = r[:, 1]
    return {
        "block": r[:, 0], "wave": hw & 0xF, "simd": (hw >> 4) & 0x3, "cu": (hw >> 8) & 0xF, "sh": (hw >> 12) & 0x1,
        "se": (hw >> 13) & 0x7, "xcc": r[:, 2] & 0xF, "ok": r[:, 3] == 0,
        "entry": r[:, 4] | (r[:, 5] << 32), "exit": r[:, 6] | (r[:, 7] << 32),
    }


def victim_axpb(x, y, a, b, stream=None):
    """The elementwise victim y = a * x + b on fp32 GPU tensors of equal size
    (tide_victim_axpb)."""
    import torch

    for t, what in ((x, "x"), (y, "y")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
            raise TypeError(f"{what}: expected a GPU torch.float32 tensor")
        if not t.is_contiguous():
            raise ValueError(f"{what}: expected a contiguous tensor")
    if x.numel() != y.numel():
        raise ValueError("x and y must have the same number of elements")
    _check(lib.tide_victim_axpb(ctypes.c_void_p(x.data_ptr() or None), ctypes.c_void_p(y.data_ptr() or None),
                                x.numel(), ctypes.c_float(a), ctypes.c_float(b),
                                ctypes.c_void_p(_stream_handle(stream) or None)))


class Stream:
    """A library-created stream (tide_stream_create), optionally restricted to
    the CUs in `cu_mask` (a sequence of CU indices).  `.torch` is the same
    stream as a torch.cuda.ExternalStream, for events and torch work."""

    def __init__(self, cus=None):
        import torch

        handle = ctypes.c_void_p()
        if cus is None:
            _check(lib.tide_stream_create(None, 0, ctypes.byref(handle)))
        else:
            n = device_info()["cu_count"]
            words = [0] * ((n + 31) // 32)
            for c in cus:
                if not 0 <= int(c) < n:
                    raise ValueError(f"CU index {c} out of range [0, {n})")
                words[int(c) // 32] |= 1 << (int(c) % 32)
            arr = (ctypes.c_uint32 * len(words))(*words)
            _check(lib.tide_stream_create(arr, len(words), ctypes.byref(handle)))
        self.handle = handle.value
        self.torch = torch.cuda.ExternalStream(self.handle)

    def destroy(self):
        if getattr(self, "handle", None):
            self.torch.synchronize()
            _check(lib.tide_stream_destroy(ctypes.c_void_p(self.handle)))
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
