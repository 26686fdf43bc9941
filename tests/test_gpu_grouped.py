"""GPU parity of coli_qgemv_grouped (int4 rows, one fp32 scale per gs
elements along I) against the fp64 oracle, through the C ABI.

Bar: |y - y_ref| <= 1e-4 * sum_g |scale[o,g]| sum_{i in g} |v(o,i) x[s,i]| + 1e-6;
bit-exact when inputs are small integers and scales powers of two."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
REL = 1e-4
GS = (32, 64, 128, 256)


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def group_scales(g, O, I, gs):
    ng = (I + gs - 1) // gs
    return synth.scales(g, O * ng).reshape(O, ng)


def run_gpu(dev, W, sc, gs, x, O):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    y = torch.full((x.shape[0], O), float("nan"), dtype=torch.float32, device=dev)
    b.qgemv_grouped(to_dev(W, dev), to_dev(sc, dev), gs, to_dev(x, dev), y, O=O)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("gs", GS)
def test_small_shapes(dev, orc, gs):
    """Short rows (one 16-byte segment) up to several k-blocks, a last group
    shorter than gs, ragged O, S up to 5 (three token passes)."""
    g = synth.rng(7100, gs)
    for O in (1, 5, 17, 40):
        for I in (32, 64, 96, 160, 288, 1000 - 1000 % 32, 2048 + 96):
            S = 1 + (O + I // 32) % 5
            announce("grouped small", gs, O, I, S)
            W = synth.weight_bytes(g, 2, O, I)
            sc = group_scales(g, O, I, gs)
            x = synth.activations(g, S, I)
            ref, mag = orc.qgemv_grouped(W, sc, gs, x)
            got = run_gpu(dev, W, sc, gs, x, O)
            assert_within(got, ref, mag, REL, what=f"gs{gs} O{O} I{I} S{S}")


@pytest.mark.parametrize("gs", GS + (384,))
def test_exact_integer_bitwise(dev, orc, gs):
    """Integer x in [-4, 4] and power-of-two scales per group: every partial
    sum is an exact fp32 value, so the device result equals the oracle's.
    Up to 2 rows one pass of the two-row kernel; from 3 rows (gs 32: from 7)
    the rounds kernel (passes of 8 rows; 9 rows: a second pass of one) while
    the block's scales fit its LDS (gs 32 at I = 12288 takes two-row passes);
    8200 rows take 32- or 48-row blocks with a ragged last one.  Both places
    of the partial tiles are met: past the staging (two-row kernel at
    I = 12288, rounds kernel with 32-row blocks at the narrow widths) and
    over it (two-row kernel at the narrow widths, rounds kernel otherwise)."""
    g = synth.rng(7200, gs)
    for O, I in ((37, 1024 + 32), (300, 4096), (64, 12288), (8200, 1024 + 128)):
        for S in (1, 2, 3, 8, 9):
            announce("grouped exact", gs, O, I, S)
            W = synth.weight_bytes(g, 2, O, I)
            ng = (I + gs - 1) // gs
            sc = synth.exact_scales(g, O * ng).reshape(O, ng)
            x = synth.exact_activations(g, S, I)
            ref, _ = orc.qgemv_grouped(W, sc, gs, x)
            got = run_gpu(dev, W, sc, gs, x, O)
            assert np.array_equal(got.astype(np.float64), ref), f"gs{gs} O{O} I{I} S{S}"


def test_group_scale_is_applied_per_group(dev, orc):
    """One group's scale set to zero removes exactly that group's elements:
    the result equals the product with x zeroed on that group."""
    g = synth.rng(7300)
    O, I, gs = 48, 1024, 32
    W = synth.weight_bytes(g, 2, O, I)
    sc = synth.exact_scales(g, O * (I // gs)).reshape(O, I // gs)
    x = synth.exact_activations(g, 2, I)
    for grp in (0, 5, 13, I // gs - 1):
        announce("grouped zero group", grp)
        s2 = sc.copy()
        s2[:, grp] = 0
        x2 = x.copy()
        x2[:, grp * gs:(grp + 1) * gs] = 0
        got = run_gpu(dev, W, s2, gs, x, O)
        want = run_gpu(dev, W, sc, gs, x2, O)
        ref, _ = orc.qgemv_grouped(W, s2, gs, x)
        assert np.array_equal(got.astype(np.float64), ref)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("gs", (32, 128))
def test_full_size_12288x6144_sampled(dev, orc, gs):
    """The dense sweep's matrix in grouped form: O=12288, I=6144, S in
    {1, 2, 4, 8}; the oracle checks 1024 sampled output rows."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    O, I = 12288, 6144
    g = synth.rng(7400, gs)
    W = synth.weight_bytes(g, 2, O, I)
    sc = group_scales(g, O, I, gs)
    Wd, scd = to_dev(W, dev), to_dev(sc, dev)
    rows = np.sort(g.choice(O, 1024, replace=False))
    rows[0], rows[-1] = 0, O - 1
    for S in (1, 2, 4, 8):
        announce("grouped 12288x6144", gs, S)
        x = synth.activations(g, S, I)
        y = torch.empty((S, O), dtype=torch.float32, device=dev)
        b.qgemv_grouped(Wd, scd, gs, to_dev(x, dev), y)
        torch.cuda.synchronize()
        got = y.cpu().numpy()[:, rows]
        ref, mag = orc.qgemv_grouped(W[rows], sc[rows], gs, x)
        assert_within(got, ref, mag, REL, what=f"gs{gs} S{S}")


def test_errors_and_empty(dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    announce("grouped errors")
    L = b.lib()
    O, I = 8, 256
    W = torch.zeros((O, I // 2), dtype=torch.uint8, device=dev)
    sc = torch.ones((O, I // 32), device=dev)
    x = torch.zeros((2, I), device=dev)
    y = torch.full((2, O), 7.0, device=dev)
    p = lambda t: t.data_ptr()
    call = lambda gs, I_, S=2, O_=O, Wp=None, xp=None: L.coli_qgemv_grouped(
        p(W) if Wp is None else Wp, p(sc), gs, p(x) if xp is None else xp, p(y), S, I_, O_, None)
    # group sizes outside {32, 64, 128k}
    for gs in (0, -1, 16, 48, 96, 200):
        assert call(gs, I) == b.ERANGE, gs
    # I not a whole number of 16-byte row segments, or past 12288
    assert call(32, 200) == b.EALIGN
    assert call(32, 12288 + 32) == b.ERANGE
    # misaligned operands
    assert call(32, I, Wp=p(W) + 4) == b.EALIGN
    assert call(32, I, xp=p(x) + 4) == b.EALIGN
    assert L.coli_qgemv_grouped(p(W), p(sc) + 4, 32, p(x), p(y), 2, I, O, None) == b.EALIGN
    # null operands
    assert L.coli_qgemv_grouped(None, p(sc), 32, p(x), p(y), 2, I, O, None) == b.EINVAL
    assert L.coli_qgemv_grouped(p(W), None, 32, p(x), p(y), 2, I, O, None) == b.EINVAL
    # S == 0 and O == 0 write nothing
    assert call(32, I, S=0) == 0
    assert call(32, I, O_=0) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
