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
