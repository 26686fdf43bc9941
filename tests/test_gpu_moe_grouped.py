"""Grouped-scale int4 experts (one scale per gs elements along a row) on the
matrix-core expert kernels.

* The pack kernels' bytes equal the grouped tiled layout and the packed
  scale layout written out here in numpy from their definitions in coli.h
  (byte work: exact).
* The MoE outputs are checked against the oracle's grouped-scale MoE (fp64,
  one scale per group) at the fp32-precision bar (1e-4) and, on the bf16
  prefill kernels, at the prefill bar (2e-2), over every group size the
  kernels specialise (32, 64, 128 and the groups of 256 or more that span
  k-blocks), ragged widths whose last group is partial, a shared expert, the
  64-token layer and the 2048-token Zipf layer."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from test_gpu_tiled import tiled_reference
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def grouped_tiled_reference(W, O, rb):
    """Row bytes [count, O, rb] -> the grouped tiled layout: each row's
    64-byte segment as 16 four-byte words, word 4 q + s taken from word
    4 s + q, then the tiled layout of those rows."""
    count = W.shape[0]
    ns = -(-rb // 64)
    pad = np.zeros((count, O, ns * 64), np.uint8)
    pad[:, :, :rb] = W
    t = pad.reshape(count, O, ns, 4, 4, 4).transpose(0, 1, 2, 4, 3, 5)   # [.., s, q, 4] -> [.., q, s, 4]
    return tiled_reference(np.ascontiguousarray(t).reshape(count, O, ns * 64), O, ns * 64)


def scales_reference(S, O, I, gs):
    """[count, O, ceil(I / gs)] -> [count, row tile, kpad / gs, 16], zero
    past O and past the last group."""
    count, ng = S.shape[0], -(-I // gs)
    mt16, ngp = -(-O // 16), -(-I // 1024) * 1024 // gs
    out = np.zeros((count, mt16 * 16, ngp), np.float32)
    out[:, :O, :ng] = S
    return out.reshape(count, mt16, 16, ngp).transpose(0, 1, 3, 2).reshape(-1)


@pytest.mark.parametrize("O,I,count", [(40, 96, 3), (130, 160, 2), (17, 2080, 2), (2048, 6144, 1)])
def test_pack_grouped_bytes(dev, O, I, count):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    g = synth.rng(6100, O, I)
    rb = b.row_bytes(2, I)
    W = g.integers(0, 256, size=(count, O, rb), dtype=np.uint8)
    announce("pack tiled grouped", O, I, count)
    got = b.pack_tiled_grouped(to_dev(W, dev), count, O, I)
    torch.cuda.synchronize()
    ref = grouped_tiled_reference(W, O, rb)
    assert got.numel() == ref.size == b.tiled_bytes(2, count, O, I)
    np.testing.assert_array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("O,I,gs,count", [(40, 96, 32, 3), (130, 160, 64, 2), (17, 1100, 1024, 2),
                                          (33, 2080, 256, 2), (2048, 6144, 128, 1)])
def test_pack_scales_bytes(dev, O, I, gs, count):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    g = synth.rng(6200, O, I, gs)
    S = np.stack([synth.group_scales(g, O, I, gs) for _ in range(count)])
    announce("pack scales grouped", O, I, gs, count)
    got = b.pack_scales_grouped(to_dev(S, dev), count, O, I, gs)
    torch.cuda.synchronize()
    ref = scales_reference(S, O, I, gs)
    assert got.numel() * 4 == ref.size * 4 == b.grouped_scale_bytes(count, O, I, gs)
    np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def _dev(d, dev):
    out = dict(d)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(d[k], dev)
    return out


@pytest.mark.parametrize("D,F,gs", [(512, 256, 32), (512, 256, 64), (512, 256, 128), (1024, 512, 256),
                                    (2048, 1024, 512), (1536, 320, 1024), (96, 160, 64), (2080, 544, 32),
                                    (1056, 800, 256)])
def test_moe_gemv_grouped(dev, orc, D, F, gs):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, S, K = 12, 23, 4
    bank = synth.expert_bank(6300 + gs, 2, E, D, F, gs=gs)
    g = synth.rng(6301, D, F, gs)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[2, 1] = -1
    td = b.tile_mlps(_dev(bank, dev))
    assert td["layout"] == b.LAYOUT_TILED_GROUPED
    announce("moe gemv grouped", D, F, gs)
    out, _ = b.moe_gemv(td, to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev))
    torch.cuda.synchronize()
    ref = orc.moe(bank, None, x, idx, w.astype(np.float64))
    assert_within(out.cpu().numpy(), ref["out"], ref["mag"], 1e-4, what=f"grouped D{D} F{F} gs{gs}")


@pytest.mark.parametrize("D,F,gs", [(512, 256, 32), (512, 256, 64), (512, 256, 128), (1024, 512, 256),
                                    (2048, 1024, 512), (96, 160, 64), (2080, 544, 32), (1056, 800, 256)])
def test_moe_gemv_grouped_bf16(dev, orc, D, F, gs):
    """The bf16 prefill kernels on grouped-scale experts (activations rounded
    once to bf16): the prefill bar, 2e-2 of the chain magnitude."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, S, K = 12, 150, 4
    bank = synth.expert_bank(6700 + gs, 2, E, D, F, gs=gs)
    g = synth.rng(6701, D, F, gs)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[2, 1] = -1
    td = b.tile_mlps(_dev(bank, dev))
    announce("moe gemv grouped bf16", D, F, gs)
    out, _ = b.moe_gemv(td, to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev), prec=b.PREC_BF16)
    torch.cuda.synchronize()
    ref = orc.moe(bank, None, x, idx, w.astype(np.float64))
    assert_within(out.cpu().numpy(), ref["out"], ref["mag"], 2e-2, what=f"grouped bf16 D{D} F{F} gs{gs}")


@pytest.mark.parametrize("gs", [32, 128])
@pytest.mark.parametrize("prec", [0, 1])
def test_moe_layer_grouped_with_shared_and_router(dev, orc, gs, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 24, 512, 256, 41, 6
    bank = synth.expert_bank(6400, 2, E, D, F, gs=gs)
    shared = synth.shared_mlp(6400, 2, D, F, gs=gs)
    g = synth.rng(6401, gs)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    td, tsd = b.tile_mlps(_dev(bank, dev)), b.tile_mlps(_dev(shared, dev), D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    announce("moe layer grouped", gs, prec)
    out, _ = b.moe_layer(rp, td, tsd, to_dev(x, dev), idx_out=idx_o, w_out=w_o, prec=prec)
    torch.cuda.synchronize()
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    ref = orc.moe(bank, shared, x, r["idx"], r["w"])
    assert_within(out.cpu().numpy(), ref["out"], ref["mag"], 2e-2 if prec else 1e-4,
                  what=f"grouped layer gs{gs} prec{prec}")
    # no integer dots on grouped experts
    with pytest.raises(b.ColiError):
        b.moe_layer(rp, td, tsd, to_dev(x, dev), prec=b.PREC_IDOT)


def _glm_grouped(glm_bank, gs, seed):
    """The 6144 x 2048 int4 bank's weights with grouped scales of gs."""
    bank, shared = glm_bank
    g = synth.rng(seed, gs)
    E, D, F = bank["E"], bank["D"], bank["F"]
    gb = dict(bank, gs=gs)
    gb["sg"] = np.stack([synth.group_scales(g, F, D, gs) for _ in range(E)])
    gb["su"] = np.stack([synth.group_scales(g, F, D, gs) for _ in range(E)])
    gb["sd"] = np.stack([synth.group_scales(g, D, F, gs) for _ in range(E)])
    gsh = dict(shared, gs=gs, sg=synth.group_scales(g, F, D, gs), su=synth.group_scales(g, F, D, gs),
               sd=synth.group_scales(g, D, F, gs))
    return gb, gsh


@pytest.mark.parametrize("gs", [32, 128])
def test_layer_64_tokens_grouped(dev, orc, glm_bank, gs):
    """The 64-token layer (256 grouped-scale int4 experts of 6144 x 2048,
    shared expert, router): within the oracle's bound on 16 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = _glm_grouped(glm_bank, gs, 6500)
    S, K, E, D = 64, 8, 256, 6144
    g = synth.rng(6501, gs)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    td, tsd = b.tile_mlps(_dev(bank, dev)), b.tile_mlps(_dev(shared, dev), D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    announce("layer 64 grouped", gs)
    out, _ = b.moe_layer(rp, td, tsd, to_dev(x, dev), idx_out=idx_o, w_out=w_o)
    torch.cuda.synchronize()
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    toks = np.sort(g.choice(S, 16, replace=False))
    ref = orc.moe(bank, shared, x[toks], r["idx"][toks], r["w"][toks])
    assert_within(out.cpu().numpy()[toks], ref["out"], ref["mag"], 1e-4, what=f"layer64 grouped gs{gs}")
    del td, tsd


def test_prefill_2048_grouped(dev, orc, glm_bank):
    """The 2048-token Zipf layer with gs = 128 group scales (fp32 precision):
    within the oracle's bound on 8 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = _glm_grouped(glm_bank, 128, 6600)
    S, K, E, D = 2048, 8, 256, 6144
    g = synth.rng(6601)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    td, tsd = b.tile_mlps(_dev(bank, dev)), b.tile_mlps(_dev(shared, dev), D)
    announce("prefill 2048 grouped")
    out, _ = b.moe_layer(None, td, tsd, to_dev(x, dev), pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev))
    torch.cuda.synchronize()
    toks = np.sort(g.choice(S, 8, replace=False))
    ref = orc.moe(bank, shared, x[toks], idx[toks], w[toks].astype(np.float64))
    assert_within(out.cpu().numpy()[toks], ref["out"], ref["mag"], 1e-4, what="prefill 2048 grouped")
    del td, tsd


@pytest.mark.parametrize("gs", [32, 128])
def test_prefill_2048_grouped_bf16(dev, orc, glm_bank, gs):
    """The 2048-token Zipf layer with grouped scales on the bf16 prefill
    kernels: within the prefill bar of the oracle on 8 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = _glm_grouped(glm_bank, gs, 6800)
    S, K, E, D = 2048, 8, 256, 6144
    g = synth.rng(6801, gs)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    td, tsd = b.tile_mlps(_dev(bank, dev)), b.tile_mlps(_dev(shared, dev), D)
    announce("prefill 2048 grouped bf16", gs)
    out, _ = b.moe_layer(None, td, tsd, to_dev(x, dev), pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev),
                         prec=b.PREC_BF16)
    torch.cuda.synchronize()
    toks = np.sort(g.choice(S, 8, replace=False))
    ref = orc.moe(bank, shared, x[toks], idx[toks], w[toks].astype(np.float64))
    assert_within(out.cpu().numpy()[toks], ref["out"], ref["mag"], 2e-2, what=f"prefill 2048 grouped bf16 gs{gs}")
    del td, tsd
