"""Helpers for the GPU parity tests (host-side comparisons only)."""
import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev())


def bf16_dev(bits):
    """uint16 numpy bf16 bits -> torch.bfloat16 on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def bf16_host(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def ordered(bits_u16):
    """bf16 bit patterns -> integers whose difference counts bf16 ulps."""
    b = bits_u16.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a, b):
    return np.abs(ordered(a) - ordered(b))


def f32_ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_isnan(bits):
    b = np.asarray(bits, np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def assert_bf16_equal(got, ref, what=""):
    """Bit-for-bit equality of bf16 outputs; where the reference is NaN the
    output must be a NaN too (sign and payload are not part of the contract).
    On failure the message names the first differing element and the largest
    difference in bf16 ulps."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    gn, rn = bf16_isnan(got), bf16_isnan(ref)
    bad = (gn != rn) | (~rn & (got != ref))
    if bad.any():
        first = tuple(int(v[0]) for v in np.nonzero(bad))
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} bf16 outputs differ; first at {first}: "
            f"got {int(got[first]):#06x}, want {int(ref[first]):#06x}; max "
            f"{int(bf16_ulp_diff(got[bad & ~gn & ~rn], ref[bad & ~gn & ~rn]).max(initial=0))} ulp")
