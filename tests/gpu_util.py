"""Helpers for the GPU tests: moving bf16 bit patterns between numpy and
torch, and comparing fp32 results bit for bit (any NaN matches any NaN)."""
import numpy as np


def to_device_bf16(bits, device="cuda"):
    import torch

    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t):
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def assert_same_f32(got, want, what=""):
    """Bitwise equality of fp32 arrays; a NaN must meet a NaN (any payload).
    Reports the maximum absolute error (0 when equal)."""
    got = np.asarray(got, dtype=np.float32).reshape(-1)
    want = np.asarray(want, dtype=np.float32).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({int((gn != wn).sum())} elements)"
    gb, wb = got.view(np.uint32)[~gn], want.view(np.uint32)[~wn]
    bad = np.nonzero(gb != wb)[0]
    if bad.size:
        i = bad[0]
        with np.errstate(invalid="ignore"):
            err = float(np.nanmax(np.abs(got[~gn].astype(np.float64) - want[~wn].astype(np.float64))))
        raise AssertionError(f"{what}: {bad.size} elements differ; first at {i}: got {gb[i]:#010x} want {wb[i]:#010x};"
                             f" max abs error {err}")
