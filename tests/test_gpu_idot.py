"""GPU parity of coli_qgemv_idot (the integer-dot qgemv: int8 activations by
absmax/127, exact integer dot, fp32 epilogue in the pages' order) against the
oracle.  Every step is integer or the same sequence of fp32 roundings, so the
bar is bit-exactness: y, the per-row activation scales and the per-row sums
of the quantised values must equal the oracle's bit for bit."""
import numpy as np
import pytest

from gpu_helpers import announce, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
I8, I4 = 1, 2


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def run(dev, fmt, W, sc, x, O):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    y = torch.full((x.shape[0], O), float("nan"), dtype=torch.float32, device=dev)
    y, ws = b.qgemv_idot(fmt, to_dev(W, dev), to_dev(sc, dev), to_dev(x, dev), y, O=O)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ws.cpu().numpy()


def ws_scales(ws, S, I):
    tb = (S * ((I + 255) // 256 * 256) + 255) // 256 * 256
    sx = np.frombuffer(ws[tb:tb + 4 * S].tobytes(), np.float32)
    sq = np.frombuffer(ws[tb + 4 * S:tb + 20 * S].tobytes(), np.int32).reshape(S, 4).sum(axis=1)
    return sx, sq


def check(orc, dev, fmt, W, sc, x, O, what):
    got, ws = run(dev, fmt, W, sc, x, O)
    ref, _ = orc.qgemv_idot(fmt, W, sc, x, O=O)
    q, s = orc.qrow_i8(x)
    sx, sq = ws_scales(ws, x.shape[0], x.shape[1])
    np.testing.assert_array_equal(sx, s, err_msg=f"{what}: row scales")
    np.testing.assert_array_equal(sq, q.astype(np.int64).sum(axis=1), err_msg=f"{what}: row sums")
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (
        f"{what}: {int((got != ref).sum())} of {got.size} differ; max |d| {np.abs(got - ref).max()}")


@pytest.mark.parametrize("fmt", [I8, I4])
@pytest.mark.parametrize("O,I", [(37, 64), (300, 1024), (129, 2048 + 64), (16, 32), (40, 96)])
def test_idot_shapes_and_passes(dev, orc, fmt, O, I):
    """Several tiles, ragged O, k-blocks past the last wave's share, rows
    shorter than 64 bytes, and 1 to 3 passes of 16 activation rows."""
    g = synth.rng(900, fmt, O, I)
    W = synth.weight_bytes(g, fmt, O, I)
    sc = synth.scales(g, O)
    for S in (1, 2, 5, 16, 17, 33):
        announce("idot", fmt, O, I, S)
        x = synth.activations(g, S, I) * np.float32(g.uniform(0.1, 10))
        check(orc, dev, fmt, W, sc, x, O, f"fmt{fmt} O{O} I{I} S{S}")


@pytest.mark.parametrize("fmt", [I8, I4])
def test_idot_extremes(dev, orc, fmt):
    """The largest width the kernels take, a zero row (scale clamp), rows whose
    quantised values hit +-127 and exact ties, and the extreme weights."""
    I = 8192 if fmt == I8 else 16384
    O = 48
    g = synth.rng(901, fmt)
    W = synth.weight_bytes(g, fmt, O, I)
    W[0] = 0x80 if fmt == I8 else 0x00          # -128 / -8 everywhere
    W[1] = 0x7F if fmt == I8 else 0xFF          # 127 / 7 everywhere
    sc = synth.scales(g, O)
    x = synth.activations(g, 4, I)
    x[1] = 0.0
    x[2] = np.round(x[2] * 4) / 4               # quarter steps: ties after scaling
    x[2, 7] = 127.0 * 4                         # s = 4: q = x / 4 exactly, ties at .5
    announce("idot extremes", fmt)
    check(orc, dev, fmt, W, sc, x, O, f"extremes fmt{fmt}")


@pytest.mark.parametrize("fmt", [I8, I4])
def test_idot_dense_12288x6144(dev, orc, fmt):
    """The dense sweep's matrix: S in {1, 4, 8}, 1536 sampled rows bit-exact."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    O, I = 12288, 6144
    g = synth.rng(902, fmt)
    W = synth.weight_bytes(g, fmt, O, I)
    sc = synth.scales(g, O)
    Wd, scd = to_dev(W, dev), to_dev(sc, dev)
    rows = np.sort(g.choice(O, 1536, replace=False))
    rows[0], rows[-1] = 0, O - 1
    for S in (1, 4, 8):
        announce("idot 12288x6144", fmt, S)
        x = synth.activations(g, S, I)
        y, _ = b.qgemv_idot(fmt, Wd, scd, to_dev(x, dev))
        torch.cuda.synchronize()
        got = y.cpu().numpy()[:, rows]
        ref, _ = orc.qgemv_idot(fmt, W[rows], sc[rows], x)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"fmt{fmt} S{S}"


def test_idot_errors_and_empty(dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    announce("idot errors")
    g = synth.rng(903)
    x = to_dev(synth.activations(g, 2, 64), dev)
    sc = torch.ones(8, device=dev)

    def status(fmt, W, xx, ws=None, O=8):
        try:
            b.qgemv_idot(fmt, W, sc, xx, O=O, ws=ws)
        except b.ColiError as e:
            return e.status
        return b.OK

    W4 = to_dev(synth.weight_bytes(g, I4, 8, 64), dev)
    assert status(3, to_dev(synth.weight_bytes(g, 3, 8, 64), dev), x) == b.EFMT
    assert status(0, torch.zeros((8, 64), device=dev), x) == b.EFMT
    x48 = to_dev(synth.activations(g, 2, 48), dev)
    assert status(I4, to_dev(synth.weight_bytes(g, I4, 8, 48), dev), x48) == b.EALIGN   # 24-byte rows
    assert status(I4, W4, x, ws=torch.zeros(16, dtype=torch.uint8, device=dev)) == b.EWORKSPACE
    big = to_dev(synth.activations(g, 1, 8192 + 128), dev)
    assert status(I8, to_dev(synth.weight_bytes(g, I8, 8, 8192 + 128), dev), big) == b.ERANGE
    y, _ = b.qgemv_idot(I4, W4, sc, torch.zeros((0, 64), device=dev),
                        y=torch.zeros((0, 8), device=dev), ws=torch.zeros(256, dtype=torch.uint8, device=dev))
    assert y.shape == (0, 8)
