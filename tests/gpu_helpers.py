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


# Smallest relative gap between neighbouring router choices seen by the
# tests, (what, gap) per checked case; printed in the session summary.
ROUTER_GAPS = []
AMBIGUOUS_REL = 2.0 ** -20


def choice_gap(sig, bias, K):
    """Smallest relative gap between neighbours among each token's K+1
    largest choices c = sig + bias (the fp32 add the router makes), exact
    ties left out (the lowest expert index settles those the same way on
    both sides).  A near tie at or inside the K-th pick could flip on a
    one-ulp difference of a score, so such a case is ambiguous."""
    c = (np.asarray(sig, np.float32) + np.asarray(bias, np.float32)[None, :]).astype(np.float64)
    n = min(K + 1, c.shape[1])
    top = -np.sort(-c, axis=1)[:, :n]
    gaps = top[:, :-1] - top[:, 1:]
    rel = np.where(gaps > 0, gaps / np.maximum(np.abs(top[:, :-1]), 1e-300), np.inf)
    return float(rel.min()) if rel.size else float("inf")


def assert_unambiguous(sig, bias, K, what):
    """Records the case's smallest choice gap and fails it as ambiguous when
    the gap is below 2^-20 of the key, never passing it silently."""
    gap = choice_gap(sig, bias, K)
    ROUTER_GAPS.append((what, gap))
    print(f"[router gap] {what}: {gap:.3e}", flush=True)
    if gap < AMBIGUOUS_REL:
        pytest.fail(f"{what}: ambiguous routing case, neighbouring choices {gap:.3e} apart "
                    f"(relative), below 2^-20")
