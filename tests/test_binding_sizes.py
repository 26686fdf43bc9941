"""The binding refuses tensors smaller than a call reads or writes, on the
host, before the library (which only sees raw pointers) is called.  CPU
tensors: every case raises before anything runs."""
import pytest
import torch

from weight_streaming_gemv_qgemv_amd import binding as b


@pytest.fixture(scope="module")
def L():
    return b.lib()


def test_qgemv_needs_o_for_flat_weights(L):
    W = torch.zeros(37748736, dtype=torch.uint8)          # a packed copy: 1-D
    x = torch.zeros((1, 6144))
    sc = torch.zeros(12288)
    with pytest.raises(b.ColiError) as e:
        b.qgemv(b.I4, W, sc, x)
    assert e.value.status == b.EINVAL
    with pytest.raises(b.ColiError) as e:                  # O given, buffer too small
        b.qgemv(b.I4, W[:1000], sc, x, O=12288)
    assert e.value.status == b.ESHAPE


def test_qgemv_short_scale_and_output(L):
    W = torch.zeros((64, 16), dtype=torch.uint8)
    x = torch.zeros((2, 32))
    with pytest.raises(b.ColiError):
        b.qgemv(b.I4, W, torch.zeros(63), x)
    with pytest.raises(b.ColiError):
        b.qgemv(b.I4, W, torch.zeros(64), x, y=torch.zeros((2, 63)))


def test_moe_sizes(L):
    E, D, F = 4, 64, 32
    ex = dict(fmt=b.I4, E=E, D=D, F=F, wg=torch.zeros((E, F, D // 2), dtype=torch.uint8),
              wu=torch.zeros((E, F, D // 2), dtype=torch.uint8),
              wd=torch.zeros((E, D, F // 2 - 1), dtype=torch.uint8),      # one byte short per row
              sg=torch.zeros((E, F)), su=torch.zeros((E, F)), sd=torch.zeros((E, D)))
    x = torch.zeros((3, D))
    idx = torch.zeros((3, 2), dtype=torch.int32)
    w = torch.zeros((3, 2))
    with pytest.raises(b.ColiError):
        b.moe_gemv(ex, x, idx, w)
    ex["wd"] = torch.zeros((E, D, F // 2), dtype=torch.uint8)
    with pytest.raises(b.ColiError):                     # x narrower than the experts
        b.moe_gemv(ex, torch.zeros((3, D - 4)), idx, w)
    with pytest.raises(b.ColiError):                     # routing shorter than S x K
        b.moe_gemv(ex, x, idx, w[:2])
    with pytest.raises(b.ColiError):                     # tiled layout: the packed size
        b.moe_gemv(dict(ex, layout=b.LAYOUT_TILED), x, idx, w)
