"""GPU parity of coli_moe_layer_tail (post-attention RMSNorm -> MoE block ->
residual add) against the oracle.

Bars:
  n:    the RMSNorm rows the device hands the block (workspace region xn)
        equal the oracle's (the pages' fp64 mean square, fp32 scale and
        products) within 1 fp32 ulp -- they differ only where the order of
        the fp64 sum moves the one rounding to fp32;
  idx:  the router's picks on the normalised rows, exactly;
  out:  |out - ref| <= rel * M + 1e-6 + 2^-22 |ref|, ref = x + block(n) in
        fp64 and M the block's chain magnitude (rel 1e-4 at fp32 precision,
        2e-2 at bf16), the last term the fp32 rounding of the residual add
        on each side.
The oracle only sees the seeded inputs and its own router's routing."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def dev_bank(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def read_xn(ws, lay, S, D):
    raw = ws.cpu().numpy()
    off = lay["xn"]
    return np.frombuffer(raw[off:off + S * D * 4].tobytes(), dtype=np.float32).reshape(S, D)


def check_tail(got, ref, rel, what):
    mag = ref["mag"] + np.abs(ref["out"]) * (2.0 ** -22 / rel)
    assert_within(got, ref["out"], mag, rel, what=what)


def check_n(n_dev, n_ref, what):
    d = np.abs(n_dev.astype(np.float64) - n_ref.astype(np.float64))
    assert np.all(d <= np.spacing(np.abs(n_ref)).astype(np.float64)), f"{what}: RMSNorm rows off by more than 1 ulp"
    return float((n_dev != n_ref).mean())


@pytest.mark.parametrize("prec", [0, 1])
def test_tail_small_with_router_and_shared(dev, orc, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 24, 512, 256, 13, 4
    bank = synth.expert_bank(80, 2, E, D, F)
    shared = synth.shared_mlp(80, 2, D, F)
    g = synth.rng(81, prec)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D) * np.float32(3.0)
    nw = g.uniform(0.5, 1.5, size=D).astype(np.float32)
    eps = 1e-5
    announce("tail small", prec)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    xd = to_dev(x, dev)
    out, ws = b.moe_layer_tail(rp, dev_bank(bank, dev), dev_bank(shared, dev), xd, to_dev(nw, dev), eps,
                               idx_out=idx_o, w_out=w_o, prec=prec)
    torch.cuda.synchronize()
    n_ref = orc.rmsnorm(x, nw, eps)
    lay = b.moe_workspace_layout(S, K, E, D, F, F, prec)
    check_n(read_xn(ws, lay, S, D), n_ref, "tail small")
    r = orc.router(Wr, bias, n_ref, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    np.testing.assert_allclose(w_o.cpu().numpy(), r["w"], rtol=1e-6)
    ref = orc.layer_tail(x, nw, eps, bank, shared, r["idx"], r["w"])
    check_tail(out.cpu().numpy(), ref, 1e-4 if prec == 0 else 2e-2, f"tail small prec{prec}")
    # in place: out is x itself, same result bit for bit
    announce("tail small in place", prec)
    x2 = xd.clone()
    b.moe_layer_tail(rp, dev_bank(bank, dev), dev_bank(shared, dev), x2, to_dev(nw, dev), eps,
                     out=x2, prec=prec, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(x2, out)


def test_tail_given_routing_vector_alu_rows(dev, orc):
    """Given routing, no shared expert, and a width whose rows are not whole
    16-byte segments (D = 501: the vector-ALU expert kernels and the scalar
    RMSNorm path)."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 501, 96, 9, 3
    bank = synth.expert_bank(82, 2, E, D, F)
    g = synth.rng(83)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    nw = g.uniform(-1.0, 2.0, size=D).astype(np.float32)
    eps = 0.25
    announce("tail given routing")
    out, ws = b.moe_layer_tail(None, dev_bank(bank, dev), None, to_dev(x, dev), to_dev(nw, dev), eps,
                               pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev))
    torch.cuda.synchronize()
    n_ref = orc.rmsnorm(x, nw, eps)
    lay = b.moe_workspace_layout(S, K, E, D, F, 0, 0)
    check_n(read_xn(ws, lay, S, D), n_ref, "tail given")
    ref = orc.layer_tail(x, nw, eps, bank, None, idx, w)
    check_tail(out.cpu().numpy(), ref, 1e-4, "tail given")


def test_tail_errors_and_empty(dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 64, 32, 3, 2
    bd = dev_bank(synth.expert_bank(84, 2, E, D, F), dev)
    g = synth.rng(85)
    x = to_dev(synth.activations(g, S, D), dev)
    idx, w = synth.routing_uniform(g, S, K, E)
    nw = torch.ones(D, device=dev)
    announce("tail errors")
    for bad_eps in (-1e-5, float("nan")):
        with pytest.raises(b.ColiError) as ei:
            b.moe_layer_tail(None, bd, None, x, nw, bad_eps, pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev))
        assert ei.value.status == b.EINVAL
    with pytest.raises(b.ColiError) as ei:
        b.moe_layer_tail(None, bd, None, x, None, 1e-5, pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev))
    assert ei.value.status == b.EINVAL
    # an empty batch enqueues nothing (empty tensors have no data pointer, so
    # the routing is left to the router)
    Wr, bias = synth.router_weights(g, E, D)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    e0 = torch.zeros((0, D), device=dev)
    o, _ = b.moe_layer_tail(rp, bd, None, e0, nw, 1e-5, out=torch.zeros((0, D), device=dev))
    assert o.shape == (0, D)


def test_tail_decode_64_tokens(dev, orc, glm_bank):
    """The 64-token decode layer as a layer tail: RMSNorm rows and router ids
    on all 64 tokens, outputs on 8 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = glm_bank
    g = synth.rng(3003)
    S, K, E, D = 64, 8, 256, 6144
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D) * np.float32(4.0)
    nw = g.uniform(0.5, 1.5, size=D).astype(np.float32)
    eps = 1e-5
    announce("tail 64 tokens")
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    out, ws = b.moe_layer_tail(rp, dev_bank(bank, dev), dev_bank(shared, dev), to_dev(x, dev),
                               to_dev(nw, dev), eps, idx_out=idx_o)
    torch.cuda.synchronize()
    n_ref = orc.rmsnorm(x, nw, eps)
    lay = b.moe_workspace_layout(S, K, E, D, 2048, 2048, 0)
    check_n(read_xn(ws, lay, S, D), n_ref, "tail 64")
    r = orc.router(Wr, bias, n_ref, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    toks = np.sort(g.choice(S, 8, replace=False))
    ref = orc.layer_tail(x[toks], nw, eps, bank, shared, r["idx"][toks], r["w"][toks])
    check_tail(out.cpu().numpy()[toks], ref, 1e-4, "tail 64")
