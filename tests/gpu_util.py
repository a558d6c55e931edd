"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def raw_pool(t, dtype):
    """Device pool -> host raw bits (uint32 for f32, uint16 otherwise)."""
    if dtype == "f32":
        return t.cpu().view(torch.int32).numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def max_abs(a, b):
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    i = np.unravel_index(np.argmax(d), d.shape) if d.size else ()
    return (float(d.max()) if d.size else 0.0), i


def bf16_rne(x):
    """float64 values rounded to bfloat16 (nearest, ties to even), as float64.
    Rounds through float32 first; the double rounding can move a value by at
    most one bf16 ulp, which the one-ulp comparisons below allow for."""
    u = np.asarray(x, np.float64).astype(np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.float64)


def bf16_ulp(x, floor=2.0 ** -14):
    """Spacing of bfloat16 numbers at max(|x|, floor) (8 significant bits).
    Below the floor (2^-14 by default) bf16's spacing is finer than the
    rounding of an fp32 sum of O(1) terms, so one ulp there is not a
    meaningful bound for any fp32 kernel; pass floor=0 for the plain spacing
    (subnormal spacing 2^-133 at the bottom)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), floor)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)
