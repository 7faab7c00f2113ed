"""Seeded generators for bf16 gradients, parameters and rank-major buffers."""
import numpy as np

from .workloads import Workload

BASE_SEED = 20261202


def bf16_bits_from_f32(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.

    NaNs stay NaNs (quiet bit set); infinities and overflow go to infinity.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)).astype(np.uint32)
    quiet = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def _normal_bf16(rng, n, sigma, outliers):
    v = rng.standard_normal(n) * sigma
    if outliers:
        mask = rng.random(n) < 0.01
        v = np.where(mask, v * 100.0, v)
    return bf16_bits_from_f32(v.astype(np.float32))


def grads_host(w: Workload, seed_index=None):
    """Rank-major list of lists: grads[u][p] = uint16 array of w.shapes[p]."""
    c = w.index if seed_index is None else seed_index
    streams = np.random.SeedSequence([BASE_SEED, c]).spawn(w.world)
    out = []
    for u in range(w.world):
        rng = np.random.Generator(np.random.PCG64(streams[u]))
        out.append([_normal_bf16(rng, w.numel(p), w.sigma, w.outliers).reshape(w.shapes[p])
                    for p in range(w.nparams)])
    return out


def params_host(w: Workload, seed_index=None):
    """Per-parameter bf16 tensors (uint16) from a stream separate from the gradients'."""
    c = w.index if seed_index is None else seed_index
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, c, 1])))
    return [_normal_bf16(rng, w.numel(p), w.sigma, False).reshape(w.shapes[p]) for p in range(w.nparams)]


def device_seed(c: int, u: int) -> int:
    """64-bit seed of rank u of workload c for torch's device generator."""
    return int(np.random.SeedSequence([BASE_SEED, c, 2, u]).generate_state(2, dtype=np.uint32).view(np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))


def grads_device(w: Workload, device, seed_index=None, dtype=None):
    """grads[u][p]: torch tensors on ``device``, generated there: bf16 (the
    default) or, with ``dtype=torch.float32``, the float32 values before the
    bf16 rounding."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype

    c = w.index if seed_index is None else seed_index
    out = []
    for u in range(w.world):
        g = torch.Generator(device=device)
        g.manual_seed(device_seed(c, u))
        row = []
        for p in range(w.nparams):
            n = w.numel(p)
            v = torch.randn(n, generator=g, device=device, dtype=torch.float32) * w.sigma
            if w.outliers:
                m = torch.rand(n, generator=g, device=device, dtype=torch.float32) < 0.01
                v = torch.where(m, v * 100.0, v)
            row.append(v.to(dtype).reshape(w.shapes[p]))
            del v
        out.append(row)
    return out


def rank_major_device(w: Workload, total_elems: int, device, seed_index=None):
    """A rank-major bf16 all-gather buffer of ``total_elems`` random values."""
    import torch

    c = w.index if seed_index is None else seed_index
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(c, 1000))
    v = torch.randn(total_elems, generator=g, device=device, dtype=torch.float32) * w.sigma
    return v.to(torch.bfloat16)
