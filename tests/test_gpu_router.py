"""GPU parity of coli_router against the oracle: expert ids bit-exact, the
fp32 sigmoid scores bit-exact (both sides take the logit in fp64 and round
once; a score may differ by one ulp only when an fp64 logit sits within
rounding distance of an fp32 midpoint, which the test counts and bounds),
weights within 1e-6 relative (fp32 normalisation on the device, fp64 in the
oracle)."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_unambiguous, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def run(dev, Wr, b, x, K, norm=1, rs=2.5, topp=0.0):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as bd
    r = bd.router(to_dev(Wr, dev), to_dev(b, dev), to_dev(x, dev), K, norm, rs, topp)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def check(got, ref, K, what, sig_ulps_allowed=2, bias=None):
    if bias is not None:
        assert_unambiguous(ref["sig"], bias, K, what)
    d = ulp_diff(got["sig"], ref["sig"])
    assert d.max() <= 1, f"{what}: a score differs by {d.max()} ulps"
    assert int((d > 0).sum()) <= sig_ulps_allowed, f"{what}: {(d > 0).sum()} scores off by 1 ulp"
    np.testing.assert_array_equal(got["idx"], ref["idx"], err_msg=what)
    np.testing.assert_array_equal(got["keff"], ref["keff"], err_msg=what)
    np.testing.assert_allclose(got["w"], ref["w"], rtol=1e-6, atol=1e-7, err_msg=what)


@pytest.mark.parametrize("E", [24, 168, 256])
@pytest.mark.parametrize("D", [64, 1000, 1001, 6144])   # 1001: unaligned rows, scalar loads
def test_router_random(dev, orc, E, D):
    g = synth.rng(515, E, D)   # seeds without a near tie (neighbouring choices >= 2^-20 apart)
    for S in (1, 7, 64, 300):            # 300: 64-token tiles, the last one ragged
        K = min(8, E)
        announce("router", E, D, S, K)
        Wr, b = synth.router_weights(g, E, D)
        x = synth.activations(g, S, D)
        ref = orc.router(Wr, b, x, K, 1, 2.5)
        got = run(dev, Wr, b, x, K)
        check(got, ref, K, f"E{E} D{D} S{S}", bias=b)


def test_router_ties_lowest_index(dev, orc):
    """Zero router weights: every score is 0.5; equal biases tie and the lower
    index wins; the weights are scores, normalised."""
    for E in (24, 168, 256, 1000):
        announce("router ties", E)
        g = synth.rng(600, E)
        D, S, K = 32, 9, 8
        Wr = np.zeros((E, D), np.float32)
        b = (g.integers(0, 3, size=E) * 0.05).astype(np.float32)   # many equal biases
        x = synth.activations(g, S, D)
        ref = orc.router(Wr, b, x, K, 1, 2.5)
        got = run(dev, Wr, b, x, K)
        check(got, ref, K, f"ties E{E}", bias=b)
        order = np.lexsort((np.arange(E), -(0.5 + b.astype(np.float64))))[:K]
        assert np.all(got["idx"] == order[None, :])


@pytest.mark.parametrize("K", [1, 2, 8, 64])
def test_router_k_range(dev, orc, K):
    g = synth.rng(700, K)
    E, D, S = 256, 256, 33
    Wr, b = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    for norm, rs in ((1, 2.5), (0, 1.0)):
        announce("router K", K, norm)
        ref = orc.router(Wr, b, x, K, norm, rs)
        got = run(dev, Wr, b, x, K, norm, rs)
        check(got, ref, K, f"K{K} norm{norm}", bias=b)


@pytest.mark.parametrize("topp", [0.3, 0.85])
def test_router_topp(dev, orc, topp):
    g = synth.rng(800)
    E, D, S, K = 256, 512, 40, 8
    Wr, b = synth.router_weights(g, E, D)
    Wr *= 8
    x = synth.activations(g, S, D)
    announce("router topp", topp)
    ref = orc.router(Wr, b, x, K, 1, 2.5, topp)
    got = run(dev, Wr, b, x, K, 1, 2.5, topp)
    check(got, ref, K, f"topp{topp}", bias=b)
    assert np.any(got["keff"] < K)


def test_router_layer_sizes(dev, orc):
    """The decode-layer router (S=64, E=256, D=6144, N(0,0.02) rows, bias
    U[-0.1,0.1]) in full, and the prefill router (S=2048) on 256 sampled
    tokens (tokens are independent)."""
    g = synth.rng(4000)
    E, D, K = 256, 6144, 8
    Wr, b = synth.router_weights(g, E, D)
    for S in (64, 2048):
        announce("router layer", S)
        x = synth.activations(g, S, D)
        got = run(dev, Wr, b, x, K)
        toks = np.arange(S) if S <= 64 else np.sort(g.choice(S, 256, replace=False))
        ref = orc.router(Wr, b, x[toks], K, 1, 2.5)
        sub = {k: v[toks] for k, v in got.items()}
        check(sub, ref, K, f"layer S{S}", bias=b)
