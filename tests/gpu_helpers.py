"""Helpers shared by the GPU parity tests."""
import sys

import numpy as np
import pytest


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    from weight_streaming_gemv_qgemv_amd import binding
    binding.lib()   # raises if libcoli.so is missing: never a silent fallback
    return torch.device("cuda:0")


def announce(*parts):
    """Name the case on stdout before a GPU step, so a crash names it."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def assert_within(got, ref, mag, rel, absol=1e-6, what=""):
    """|got - ref| <= rel * mag + absol, elementwise; reports the worst ratio."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.asarray(mag, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = rel * mag + absol
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    assert np.all(err <= bound), (
        f"{what}: {int((err > bound).sum())} of {err.size} outside tolerance; worst at {worst}: "
        f"got {got[worst]!r} ref {ref[worst]!r} bound {bound[worst]!r}")
    return float(ratio.max()) if ratio.size else 0.0
