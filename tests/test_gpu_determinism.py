"""Run-to-run determinism of the MoE layer on the matrix-core paths: the
same inputs give the same output bits on every call (fixed summation
orders, no atomics; and no stage reads data another wave has not finished
writing -- a miscounted wait before a barrier shows here as a few rows that
differ in a small fraction of calls)."""
import numpy as np
import pytest

from gpu_helpers import announce, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
REPS = 120


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _dev_bank(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


@pytest.mark.parametrize("fmt,prec", [(1, 2), (2, 2), (1, 1), (2, 1), (2, 0)])
def test_layer_bits_repeat(dev, fmt, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 16, 1024, 512, 4
    S = 64 if prec == 0 else 300
    bank = synth.expert_bank(90 + fmt, fmt, E, D, F)
    shared = synth.shared_mlp(90 + fmt, fmt, D, F)
    g = synth.rng(91, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    td = b.tile_mlps(_dev_bank(bank, dev))
    tsd = b.tile_mlps(_dev_bank(shared, dev), D)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, E, D, F, F, prec), dev)
    announce("determinism", fmt, prec)
    first = None
    differ = 0
    for _ in range(REPS):
        out, _ = b.moe_layer(None, td, tsd, xd, pre_idx=idd, pre_w=wd, prec=prec, ws=ws)
        o = out.cpu().numpy()
        if first is None:
            first = o
        elif not np.array_equal(o.view(np.uint32), first.view(np.uint32)):
            differ += 1
    torch.cuda.synchronize()
    assert differ == 0, f"{differ} of {REPS - 1} repeats differ"


@pytest.mark.parametrize("gs,prec", [(32, 0), (128, 0), (512, 0), (32, 1), (64, 1), (128, 1), (512, 1)])
def test_grouped_layer_bits_repeat(dev, gs, prec):
    """Grouped-scale int4 experts (the fp32 and bf16 kernels with the group
    scales staged beside the activations)."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 16, 1024, 512, 4
    S = 64 if prec == 0 else 300
    bank = synth.expert_bank(95, 2, E, D, F, gs=gs)
    shared = synth.shared_mlp(95, 2, D, F, gs=gs)
    g = synth.rng(96, gs)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    td = b.tile_mlps(_dev_bank(bank, dev))
    tsd = b.tile_mlps(_dev_bank(shared, dev), D)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    ws = b.alloc_workspace(b.moe_workspace_bytes(S, K, E, D, F, F, prec), dev)
    announce("determinism grouped", gs, prec)
    first = None
    differ = 0
    for _ in range(REPS):
        out, _ = b.moe_layer(None, td, tsd, xd, pre_idx=idd, pre_w=wd, ws=ws, prec=prec)
        o = out.cpu().numpy()
        if first is None:
            first = o
        elif not np.array_equal(o.view(np.uint32), first.view(np.uint32)):
            differ += 1
    torch.cuda.synchronize()
    assert differ == 0, f"{differ} of {REPS - 1} repeats differ"
