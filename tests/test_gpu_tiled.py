"""The tiled weight layout (coli_pack_tiled) on the GPU.

* The pack kernel's bytes equal the layout written out here in numpy from
  its definition in coli.h (byte work: exact).
* The expert kernels reading tiled weights do the same arithmetic in the
  same order as on the row-major weights, so the outputs agree bit for bit;
  the tiled results are also checked against the oracle (the row-major
  weights are what the oracle reads)."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def tiled_reference(W, O, rb):
    """[count, O, rb] row-major bytes -> the tiled layout: 1 KB units of 16
    rows x 64 bytes, lane 16 q + c = row c's bytes 16 q .. 16 q + 15 of the
    segment; units by groups of 8 row tiles, then segment, then row tile."""
    count = W.shape[0]
    ns, mt16 = -(-rb // 64), -(-O // 16)
    pad = np.zeros((count, mt16 * 16, ns * 64), np.uint8)
    pad[:, :O, :rb] = W
    # [count, m, c, g, q, 16] -> unit (m, g) lanes (q, c)
    u = pad.reshape(count, mt16, 16, ns, 4, 16).transpose(0, 1, 3, 4, 2, 5)   # count, m, g, q, c, 16
    out = np.zeros((count, mt16 * ns, 1024), np.uint8)
    for m in range(mt16):
        T, mm = divmod(m, 8)
        nT = min(8, mt16 - 8 * T)
        for g in range(ns):
            out[:, T * 8 * ns + g * nT + mm] = u[:, m, g].reshape(count, 1024)
    return out.reshape(-1)


@pytest.mark.parametrize("fmt,O,I,count", [(2, 40, 96, 3), (2, 130, 160, 2), (1, 17, 96, 2),
                                           (3, 160, 320, 2), (2, 2048, 6144, 1), (1, 6144, 2048, 1)])
def test_pack_bytes(dev, fmt, O, I, count):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    g = synth.rng(5100, fmt, O, I)
    rb = b.row_bytes(fmt, I)
    W = g.integers(0, 256, size=(count, O, rb), dtype=np.uint8)
    announce("pack tiled", fmt, O, I, count)
    got = b.pack_tiled(fmt, to_dev(W, dev), count, O, I)
    torch.cuda.synchronize()
    ref = tiled_reference(W, O, rb)
    assert got.numel() == ref.size == b.tiled_bytes(fmt, count, O, I)
    np.testing.assert_array_equal(got.cpu().numpy(), ref)


def _dev(d, dev):
    out = dict(d)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(d[k], dev)
    return out


def _same_bits(a, b, what):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    assert np.all(np.isfinite(a)), what
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32), err_msg=what)


@pytest.mark.parametrize("fmt,D,F", [(1, 512, 256), (2, 512, 256), (3, 512, 256),
                                     (2, 96, 160), (1, 96, 160), (3, 192, 320)])
@pytest.mark.parametrize("prec", [0, 1])
def test_moe_gemv_tiled_equals_rows(dev, orc, fmt, D, F, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, S, K = 12, 23, 4
    bank = synth.expert_bank(5200 + fmt, fmt, E, D, F)
    g = synth.rng(5201, fmt, D)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[2, 1] = -1
    bd = _dev(bank, dev)
    td = b.tile_mlps(bd)
    announce("moe gemv tiled", fmt, D, F, prec)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    o_rows, _ = b.moe_gemv(bd, xd, idd, wd, prec=prec)
    o_tiled, _ = b.moe_gemv(td, xd, idd, wd, prec=prec)
    torch.cuda.synchronize()
    _same_bits(o_tiled.cpu().numpy(), o_rows.cpu().numpy(), f"fmt{fmt} D{D} F{F} prec{prec}")
    ref = orc.moe(bank, None, x, idx, w.astype(np.float64))
    assert_within(o_tiled.cpu().numpy(), ref["out"], ref["mag"], 2e-2 if prec else 1e-4, what="tiled vs oracle")


@pytest.mark.parametrize("prec", [0, 1])
def test_moe_layer_tiled_with_shared_and_router(dev, orc, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 24, 512, 256, 41, 6
    bank = synth.expert_bank(5300, 2, E, D, F)
    shared = synth.shared_mlp(5300, 2, D, F)
    g = synth.rng(5301, prec)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    bd, sd = _dev(bank, dev), _dev(shared, dev)
    td, tsd = b.tile_mlps(bd), b.tile_mlps(sd, D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    announce("moe layer tiled", prec)
    xd = to_dev(x, dev)
    o_rows, _ = b.moe_layer(rp, bd, sd, xd, prec=prec)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    o_tiled, _ = b.moe_layer(rp, td, tsd, xd, idx_out=idx_o, w_out=w_o, prec=prec)
    torch.cuda.synchronize()
    _same_bits(o_tiled.cpu().numpy(), o_rows.cpu().numpy(), f"layer prec{prec}")
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    ref = orc.moe(bank, shared, x, r["idx"], r["w"])
    assert_within(o_tiled.cpu().numpy(), ref["out"], ref["mag"], 2e-2 if prec else 1e-4, what="tiled layer")
    # a tiled shared expert beside row-major routed experts is refused
    with pytest.raises(b.ColiError):
        b.moe_layer(rp, bd, tsd, xd, prec=prec)


def test_layer_64_tokens_tiled(dev, orc, glm_bank):
    """The 64-token layer (256 int4 experts of 6144 x 2048, shared expert,
    router) on tiled weights: bit for bit the row-major result, and within
    the bound of the oracle on 16 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = glm_bank
    S, K, E, D = 64, 8, 256, 6144
    g = synth.rng(5400)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    bd, sd = _dev(bank, dev), _dev(shared, dev)
    td, tsd = b.tile_mlps(bd), b.tile_mlps(sd, D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    xd = to_dev(x, dev)
    announce("layer 64 tiled")
    o_rows, _ = b.moe_layer(rp, bd, sd, xd)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    o_tiled, _ = b.moe_layer(rp, td, tsd, xd, idx_out=idx_o, w_out=w_o)
    torch.cuda.synchronize()
    _same_bits(o_tiled.cpu().numpy(), o_rows.cpu().numpy(), "layer64 tiled")
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    toks = np.sort(g.choice(S, 16, replace=False))
    ref = orc.moe(bank, shared, x[toks], r["idx"][toks], r["w"][toks])
    assert_within(o_tiled.cpu().numpy()[toks], ref["out"], ref["mag"], 1e-4, what="layer64 tiled")
    del td, tsd


def test_prefill_2048_tiled(dev, glm_bank):
    """The 2048-token Zipf layer in bf16 on tiled weights: bit for bit the
    row-major result (whose oracle parity the prefill tests check)."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = glm_bank
    S, K, E, D = 2048, 8, 256, 6144
    g = synth.rng(5500)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    bd, sd = _dev(bank, dev), _dev(shared, dev)
    td, tsd = b.tile_mlps(bd), b.tile_mlps(sd, D)
    xd, idd, wd = to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev)
    announce("prefill 2048 tiled")
    o_rows, _ = b.moe_layer(None, bd, sd, xd, pre_idx=idd, pre_w=wd, prec=1)
    o_tiled, _ = b.moe_layer(None, td, tsd, xd, pre_idx=idd, pre_w=wd, prec=1)
    torch.cuda.synchronize()
    _same_bits(o_tiled.cpu().numpy(), o_rows.cpu().numpy(), "prefill tiled")
