"""coli_moe_layer_noalloc -- the MoE layer on the library's static scratch,
for callers that cannot allocate -- against coli_moe_layer on the same
inputs.  Both run the same kernels in a fixed order, so the routing and the
output must agree bit for bit; two calls in a row, the second smaller, show
that nothing left in the shared scratch by one call leaks into the next."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _bank_dev(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def _both(dev, rp, bd, sd, x_np, K, prec=0, pre_idx=None, pre_w=None):
    """(out, idx, w) of coli_moe_layer and of coli_moe_layer_noalloc."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    S, D = x_np.shape
    x = to_dev(x_np, dev)
    pi = to_dev(pre_idx, dev) if pre_idx is not None else None
    pw = to_dev(pre_w, dev) if pre_w is not None else None
    idx_a = torch.full((S, K), -7, dtype=torch.int32, device=dev)
    w_a = torch.full((S, K), float("nan"), device=dev)
    out_a, _ = b.moe_layer(rp, bd, sd, x, pre_idx=pi, pre_w=pw, idx_out=idx_a, w_out=w_a, prec=prec, K=K)
    out_n = torch.full((S, D), float("nan"), device=dev)
    idx_n = torch.full((S, K), -7, dtype=torch.int32, device=dev)
    w_n = torch.full((S, K), float("nan"), device=dev)
    rc = b.moe_layer_noalloc(rp, bd, sd, x, out_n, pre_idx=pi, pre_w=pw, idx_out=idx_n, w_out=w_n,
                             prec=prec, K=K)
    assert rc == b.OK, b.strerror(rc)
    torch.cuda.synchronize()
    return [(t.cpu().numpy()) for t in (out_a, idx_a, w_a, out_n, idx_n, w_n)]


def _same(res, what):
    out_a, idx_a, w_a, out_n, idx_n, w_n = res
    np.testing.assert_array_equal(idx_n, idx_a, err_msg=what)
    np.testing.assert_array_equal(w_n.view(np.uint32), w_a.view(np.uint32), err_msg=what)
    assert np.all(np.isfinite(out_n)), what
    np.testing.assert_array_equal(out_n.view(np.uint32), out_a.view(np.uint32), err_msg=what)


@pytest.mark.parametrize("prec", [0, 1])
def test_noalloc_small_two_calls(dev, orc, prec):
    E, D, F, K = 24, 512, 256, 4
    bank = synth.expert_bank(90, 2, E, D, F)
    shared = synth.shared_mlp(90, 2, D, F)
    g = synth.rng(91, prec)
    Wr, bias = synth.router_weights(g, E, D)
    bd, sd = _bank_dev(bank, dev), _bank_dev(shared, dev)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    for S in (40, 9):
        x = synth.activations(g, S, D)
        announce("noalloc small", prec, S)
        res = _both(dev, rp, bd, sd, x, K, prec)
        _same(res, f"small prec{prec} S{S}")
        r = orc.router(Wr, bias, x, K, 1, 2.5)
        ref = orc.moe(bank, shared, x, r["idx"], r["w"])
        assert_within(res[3], ref["out"], ref["mag"], 2e-2 if prec else 1e-4, what=f"noalloc S{S}")
    # given routing (the ids and weights are copied to idx_out / w_out)
    S = 17
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    announce("noalloc given routing", prec, S)
    _same(_both(dev, None, bd, sd, x, K, prec, pre_idx=idx, pre_w=w), f"given prec{prec}")


@pytest.mark.parametrize("gs", [32, 128])
@pytest.mark.parametrize("prec", [0, 1])
def test_noalloc_grouped_scales_two_calls(dev, orc, gs, prec):
    """Grouped-scale int4 experts (grouped tiled layout, fp32 or bf16
    precision) through the static scratch: bit for bit coli_moe_layer, and
    within the oracle's bound."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 24, 512, 256, 4
    bank = synth.expert_bank(93, 2, E, D, F, gs=gs)
    shared = synth.shared_mlp(93, 2, D, F, gs=gs)
    g = synth.rng(94, gs)
    Wr, bias = synth.router_weights(g, E, D)
    td, tsd = b.tile_mlps(_bank_dev(bank, dev)), b.tile_mlps(_bank_dev(shared, dev), D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    for S in (40, 9):
        x = synth.activations(g, S, D)
        announce("noalloc grouped", gs, prec, S)
        res = _both(dev, rp, td, tsd, x, K, prec)
        _same(res, f"grouped gs{gs} prec{prec} S{S}")
        r = orc.router(Wr, bias, x, K, 1, 2.5)
        ref = orc.moe(bank, shared, x, r["idx"], r["w"])
        assert_within(res[3], ref["out"], ref["mag"], 2e-2 if prec else 1e-4,
                      what=f"noalloc grouped gs{gs} prec{prec} S{S}")


@pytest.mark.parametrize("fmt", [1, 2])
def test_noalloc_integer_dots_two_calls(dev, fmt):
    """The integer-dot expert path (tiled int8 / int4) through the static
    scratch: bit for bit coli_moe_layer on the same inputs."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 24, 512, 256, 4
    bank = synth.expert_bank(95, fmt, E, D, F)
    shared = synth.shared_mlp(95, fmt, D, F)
    g = synth.rng(96, fmt)
    Wr, bias = synth.router_weights(g, E, D)
    td, tsd = b.tile_mlps(_bank_dev(bank, dev)), b.tile_mlps(_bank_dev(shared, dev), D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    for S in (40, 9):
        x = synth.activations(g, S, D)
        announce("noalloc idot", fmt, S)
        _same(_both(dev, rp, td, tsd, x, K, prec=b.PREC_IDOT), f"idot fmt{fmt} S{S}")


def test_noalloc_layer_64_then_16_tokens(dev, glm_bank):
    """The 64-token layer (router, 256 int4 experts of 6144 x 2048, shared
    expert), then 16 tokens, through the static scratch."""
    bank, shared = glm_bank
    E, D, K = 256, 6144, 8
    g = synth.rng(92)
    Wr, bias = synth.router_weights(g, E, D)
    bd, sd = _bank_dev(bank, dev), _bank_dev(shared, dev)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    for S in (64, 16):
        x = synth.activations(g, S, D)
        announce("noalloc layer", S)
        _same(_both(dev, rp, bd, sd, x, K), f"layer S{S}")


def test_noalloc_refuses_sizes_past_the_scratch(dev):
    """A batch whose workspace exceeds the static scratch is refused before
    any device work (300 tokens of the 256 x 6144/2048 layer need ~133 MiB)."""
    import ctypes as C
    from weight_streaming_gemv_qgemv_amd import binding as b
    FAKE = 0x10000
    ex = b.Experts(2, 256, 6144, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    sh = b.Mlp(2, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    rp = b.RouterParams(FAKE, FAKE, 8, 1, 2.5, 0.0)
    assert b.moe_workspace_bytes(300, 8, 256, 6144, 2048, 2048) > (64 << 20)
    rc = b.lib().coli_moe_layer_noalloc(C.byref(rp), C.byref(ex), C.byref(sh), FAKE, 300, None, None, FAKE,
                                        None, None, 0, None)
    assert rc == b.ERANGE
