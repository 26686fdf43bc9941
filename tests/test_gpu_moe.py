"""GPU parity of coli_moe_gemv / coli_moe_layer against the oracle.

Bars (COLI_PREC_FP32):
  out:  |out - ref| <= 1e-4 * M_out + 1e-6, M_out = sum_k |w_k| |sd[o]| sum_j
        |vd(o,j) h_j| (+ the shared expert's term): the per-product bound of
        the last contraction, weighted as it is combined;
  h:    the SwiGLU output per grouped row, against the oracle's h with the
        first-order propagation of the gate/up bounds:
        1e-4 * (1.1 * Mg |u| + |silu(g)| Mu) + 1e-6;
  y:    each expert's down output per grouped row, against the oracle's
        down product of the oracle's h, with the down product's own bound
        plus the h bound carried through |sd vd|.
Expert ids and grouping are integers: checked exactly.  The oracle only ever
sees the seeded inputs (and, for the layer tests, its own router's routing),
never a device result."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_unambiguous, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
REL = 1e-4


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def dev_bank(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def silu(z):
    return z / (1.0 + np.exp(-z))


def read_ws(ws, lay, S, K, D, Fld, rows):
    raw = ws.cpu().numpy()

    def arr(off, n, dt):
        return np.frombuffer(raw[off:off + n * np.dtype(dt).itemsize].tobytes(), dtype=dt)

    P = S * K
    return dict(
        flags=int(arr(lay["flags"], 1, np.uint32)[0]),
        pair_row=arr(lay["pair_row"], P, np.int32),
        row_pair=arr(lay["row_pair"], P, np.int32),
        h=arr(lay["h"], rows * Fld, np.float32).reshape(rows, Fld),
        y=arr(lay["y"], rows * D, np.float32).reshape(rows, D),
    )


def check_moe(orc, bank, shared, x, idx, w, out, ws, lay, what, rel=REL):
    S, K = idx.shape
    D, F = bank["D"], bank["F"]
    ref = orc.moe(bank, shared, x, idx, w.astype(np.float64), intermediates=True)
    assert_within(out, ref["out"], ref["mag"], rel, what=what + " out")
    rows = S * K + (S if shared is not None else 0)
    wsd = read_ws(ws, lay, S, K, D, lay["h_ld"], rows)
    # grouping: pair_row is a bijection onto the kept slots, ordered by expert
    # then slot
    valid = (idx.reshape(-1) >= 0) & (idx.reshape(-1) < bank["E"])
    pr = wsd["pair_row"]
    assert np.all(pr[~valid] == -1)
    kept = np.nonzero(valid)[0]
    order = kept[np.lexsort((kept, idx.reshape(-1)[kept]))]
    np.testing.assert_array_equal(pr[order], np.arange(len(order)))
    np.testing.assert_array_equal(wsd["row_pair"][:len(order)], order)
    # h per kept slot, and y from the oracle's h: the down product's bound
    # plus the h bound (rel * hb + 1e-6 per element) carried through |sd vd|
    def y_bound(fmt, wd, sd, h_ref, hb):
        _, ymag = orc.qgemv(fmt, wd, sd, h_ref[None, :])
        _, hmag = orc.qgemv(fmt, wd, sd, hb[None, :])
        _, ones = orc.qgemv(fmt, wd, sd, np.ones((1, hb.size)))
        return ymag[0] + hmag[0] + ones[0] * (1e-6 / rel)

    for p in kept[:: max(1, len(kept) // 64)]:
        r = pr[p]
        hg = wsd["h"][r, :F]
        g, u = ref["g"][p], ref["u"][p]
        bound_mag = 1.1 * ref["gmag"][p] * np.abs(u) + np.abs(silu(g)) * ref["umag"][p]
        assert_within(hg, ref["h"][p], bound_mag, rel, what=f"{what} h slot {p}")
        e = idx.reshape(-1)[p]
        yb = y_bound(bank["fmt"], bank["wd"][e], bank["sd"][e], ref["h"][p], bound_mag)
        assert_within(wsd["y"][r], ref["y"][p], yb, rel, what=f"{what} y slot {p}")
    if shared is not None and shared["F"] == F:
        for s in range(0, S, max(1, S // 8)):
            p = S * K + s
            r = p
            g, u = ref["g"][p], ref["u"][p]
            bound_mag = 1.1 * ref["gmag"][p] * np.abs(u) + np.abs(silu(g)) * ref["umag"][p]
            assert_within(wsd["h"][r, :F], ref["h"][p], bound_mag, rel, what=f"{what} shared h {s}")
            yb = y_bound(shared["fmt"], shared["wd"], shared["sd"], ref["h"][p], bound_mag)
            assert_within(wsd["y"][r], ref["y"][p], yb, rel, what=f"{what} shared y {s}")
    return wsd


def run_gemv(dev, bank_d, x, idx, w, prec=0):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    out, ws = b.moe_gemv(bank_d, to_dev(x, dev), to_dev(idx, dev), to_dev(w, dev), prec=prec)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_moe_gemv_tiny_unaligned(dev, orc, fmt):
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 6, 40, 24, 5, 3
    bank = synth.expert_bank(10 + fmt, fmt, E, D, F)
    g = synth.rng(11, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    announce("moe tiny", fmt)
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, E, D, F)
    wsd = check_moe(orc, bank, None, x, idx, w, out, ws, lay, f"tiny fmt{fmt}")
    assert wsd["flags"] == 0


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_moe_gemv_tiles_aligned(dev, orc, fmt):
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 16, 512, 256, 21, 4
    bank = synth.expert_bank(20 + fmt, fmt, E, D, F)
    g = synth.rng(21, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    idx[0, :] = [3, 4, 5, 6]
    # one expert with 20 rows: two token passes, the second partial, with a
    # dead second N-tile (passes of 16 rows as two 8-row tiles)
    for s in range(1, 20):
        row = [3] + [e for e in g.permutation(E) if e != 3][:K - 1]
        idx[s] = row
    announce("moe tiles", fmt)
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, E, D, F)
    check_moe(orc, bank, None, x, idx, w, out, ws, lay, f"tiles fmt{fmt}")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_moe_gemv_short_rows_matrix_cores(dev, orc, fmt):
    """Widths whose rows are whole 16-byte segments but shorter than 64
    bytes (int4 D=64, F=32: 32- and 16-byte rows) take the matrix-core
    kernels with their chunk offsets clamped inside the row."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 64, 32, 10, 3
    bank = synth.expert_bank(30 + fmt, fmt, E, D, F)
    g = synth.rng(31, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    announce("moe short rows", fmt)
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, E, D, F)
    check_moe(orc, bank, None, x, idx, w, out, ws, lay, f"short fmt{fmt}")


def test_moe_gemv_skipped_and_bad_slots(dev, orc):
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 256, 128, 6, 3
    bank = synth.expert_bank(30, 2, E, D, F)
    g = synth.rng(31)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_uniform(g, S, K, E)
    idx[0, 2] = -1                 # empty slot: skipped, no flag
    announce("moe skipped slot")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, E, D, F)
    check_moe(orc, bank, None, x, idx, w, out, ws, lay, "skipped")
    assert b.check_device_flags(ws) == (b.OK, 0)
    bad = idx.copy()
    bad[1, 0] = E + 3              # out of range: skipped and flagged
    bad[2, 1] = -7
    announce("moe bad ids")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, bad, w)
    rc, flags = b.check_device_flags(ws)
    assert rc == b.EIDX and flags & 1
    masked = bad.copy()
    masked[(masked < 0) | (masked >= E)] = -1
    ref = orc.moe(bank, None, x, masked, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what="bad ids")
    dup = idx.copy()
    dup[3, 1] = dup[3, 0]          # listed twice: computed twice and flagged
    announce("moe duplicate id")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, dup, w)
    rc, flags = b.check_device_flags(ws)
    assert rc == b.EIDX and flags & 2
    ref = orc.moe(bank, None, x, dup, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what="dup")


def test_moe_gemv_chunked_grouping(dev, orc):
    """More than 1024 slots take the chunked grouping: 400 tokens x 3 slots
    (two chunks; token 341's slots 1023-1025 straddle the boundary), skewed
    routing, empty slots; then a bad id and a duplicate across the boundary
    are skipped / computed twice and flagged."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 40, 256, 128, 400, 3
    bank = synth.expert_bank(32, 2, E, D, F)
    g = synth.rng(33)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[5, 1] = -1
    idx[350, 2] = -1
    announce("moe chunked grouping")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, E, D, F)
    check_moe(orc, bank, None, x, idx, w, out, ws, lay, "chunked")
    assert b.check_device_flags(ws) == (b.OK, 0)
    bad = idx.copy()
    bad[10, 0] = E + 1
    bad[341, 1] = bad[341, 0]      # slot 1024 repeats slot 1023
    announce("moe chunked grouping, bad and duplicate ids")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, bad, w)
    rc, flags = b.check_device_flags(ws)
    assert rc == b.EIDX and flags & 1 and flags & 2
    masked = bad.copy()
    masked[(masked < 0) | (masked >= E)] = -1
    ref = orc.moe(bank, None, x, masked, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what="chunked bad/dup")


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_moe_gemv_one_launch_grouping_limit(dev, orc, fmt):
    """The one-launch grouping (which also writes x's row tables) at its
    largest batch, 128 tokens x 8 slots = 1024 slots, and one token more
    (1032 slots: the chunked grouping and the separate row-table kernel);
    skewed routing with empty slots, and a bad id in the last slot."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 36, 256, 128, 8
    bank = synth.expert_bank(60 + fmt, fmt, E, D, F)
    bd = dev_bank(bank, dev)
    for S in (128, 129):
        g = synth.rng(61, fmt, S)
        x = synth.activations(g, S, D)
        idx, w = synth.routing_zipf(g, S, K, E)
        idx[3, 2] = -1
        idx[S - 1, 5] = -1
        announce("moe grouping limit", fmt, S)
        out, ws = run_gemv(dev, bd, x, idx, w)
        lay = b.moe_workspace_layout(S, K, E, D, F)
        check_moe(orc, bank, None, x, idx, w, out, ws, lay, f"limit S{S}")
        assert b.check_device_flags(ws) == (b.OK, 0)
        bad = idx.copy()
        bad[S - 1, K - 1] = E
        announce("moe grouping limit, bad id", fmt, S)
        out, ws = run_gemv(dev, bd, x, bad, w)
        rc, flags = b.check_device_flags(ws)
        assert rc == b.EIDX and flags & 1
        masked = bad.copy()
        masked[(masked < 0) | (masked >= E)] = -1
        ref = orc.moe(bank, None, x, masked, w.astype(np.float64))
        assert_within(out, ref["out"], ref["mag"], REL, what=f"limit bad S{S}")


def test_moe_layer_small_with_router_and_shared(dev, orc):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 24, 512, 256, 13, 4
    bank = synth.expert_bank(40, 2, E, D, F)
    shared = synth.shared_mlp(40, 2, D, F)
    g = synth.rng(41)
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    announce("moe layer small")
    bd = dev_bank(bank, dev)
    sd = dev_bank(shared, dev)
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    out, ws = b.moe_layer(rp, bd, sd, to_dev(x, dev), idx_out=idx_o, w_out=w_o)
    torch.cuda.synchronize()
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    np.testing.assert_allclose(w_o.cpu().numpy(), r["w"], rtol=1e-6)
    lay = b.moe_workspace_layout(S, K, E, D, F, F)
    check_moe(orc, bank, shared, x, r["idx"], r["w"], out.cpu().numpy(), ws, lay, "layer small")
    # shared only: all routed weights zero
    announce("moe layer shared only")
    z = np.zeros((S, K), np.float32)
    out2, _ = b.moe_layer(None, bd, sd, to_dev(x, dev), pre_idx=to_dev(r["idx"], dev),
                          pre_w=to_dev(z, dev))
    torch.cuda.synchronize()
    ref = orc.moe(bank, shared, x, r["idx"], z.astype(np.float64))
    assert_within(out2.cpu().numpy(), ref["out"], ref["mag"], REL, what="shared only")


def run_layer_topp(dev, bank_d, shared_d, Wr, bias, x, K, topp):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    S = x.shape[0]
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5, topp=topp)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    out, ws = b.moe_layer(rp, bank_d, shared_d, to_dev(x, dev), idx_out=idx_o, w_out=w_o)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx_o.cpu().numpy(), w_o.cpu().numpy(), ws


def check_topp_routing(orc, Wr, bias, x, K, topp, idx, w, what):
    """The router's ragged top-p output as the layer used it: ids (with -1
    past keff) exact, keff below K for some tokens, weights within 1e-6."""
    r = orc.router(Wr, bias, x, K, 1, 2.5, topp)
    assert_unambiguous(r["sig"], bias, K, what)
    np.testing.assert_array_equal(idx, r["idx"], err_msg=what)
    keff = (idx >= 0).sum(axis=1)
    np.testing.assert_array_equal(keff, r["keff"], err_msg=what)
    assert np.all(idx[np.arange(K)[None, :] >= keff[:, None]] == -1)
    assert np.any(keff < K), f"{what}: no token was truncated"
    np.testing.assert_allclose(w, r["w"], rtol=1e-6, atol=1e-7, err_msg=what)
    return r


@pytest.mark.parametrize("topp", [0.3, 0.85])
def test_moe_layer_topp_small(dev, orc, topp):
    """coli_moe_layer with top-p routing (glm.c@98759bf -- moe, phase A,
    TOPP): the router's ragged keff feeds the grouping, the products and the
    combine in one call; out against the oracle's block on the oracle's
    truncated routing, intermediates and grouping included."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 24, 512, 256, 37, 6
    bank = synth.expert_bank(42, 2, E, D, F)
    shared = synth.shared_mlp(42, 2, D, F)
    g = synth.rng(43, int(topp * 100))
    Wr, bias = synth.router_weights(g, E, D)
    Wr *= 8     # logits of a few units: the top scores spread, keff varies
    x = synth.activations(g, S, D)
    announce("moe layer topp small", topp)
    out, idx, w, ws = run_layer_topp(dev, dev_bank(bank, dev), dev_bank(shared, dev), Wr, bias, x, K, topp)
    r = check_topp_routing(orc, Wr, bias, x, K, topp, idx, w, f"topp{topp} small")
    lay = b.moe_workspace_layout(S, K, E, D, F, F)
    check_moe(orc, bank, shared, x, r["idx"], r["w"], out, ws, lay, f"layer topp{topp}")
    assert b.check_device_flags(ws) == (b.OK, 0)


def test_moe_layer_empty_batch(dev):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    announce("moe empty")
    E, D, F = 8, 64, 32
    bd = dev_bank(synth.expert_bank(50, 2, E, D, F), dev)
    x = torch.zeros((0, D), device=dev)
    out = torch.zeros((0, D), device=dev)
    idx = torch.zeros((0, 2), dtype=torch.int32, device=dev)
    w = torch.zeros((0, 2), device=dev)
    o, _ = b.moe_gemv(bd, x, idx, w, out=out)
    assert o.shape == (0, D)


# ---------------------------------------------------------------- full size
# (the glm_bank fixture -- 256 int4 experts of 6144 x 2048 plus the shared
# expert -- lives in conftest.py, shared with the prefill tests)
def test_expert_decode_16_tokens(dev, orc, glm_bank):
    """256 int4 experts, 16 tokens, given top-8 routing: full oracle check."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, _ = glm_bank
    g = synth.rng(3001)
    S, K = 16, 8
    x = synth.activations(g, S, 6144)
    idx, w = synth.routing_uniform(g, S, K, 256)
    announce("moe decode 16 tokens")
    out, ws = run_gemv(dev, dev_bank(bank, dev), x, idx, w)
    lay = b.moe_workspace_layout(S, K, 256, 6144, 2048)
    check_moe(orc, bank, None, x, idx, w, out, ws, lay, "decode16")


def test_layer_decode_64_tokens(dev, orc, glm_bank):
    """Full layer, 64 ragged decode rows: router + 256 int4 experts + shared;
    ids exact on all 64 tokens, outputs checked on 16 sampled tokens."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    bank, shared = glm_bank
    g = synth.rng(3002)
    S, K, E, D = 64, 8, 256, 6144
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    announce("moe layer 64 tokens")
    rp = dict(w=to_dev(Wr, dev), bias=to_dev(bias, dev), K=K, norm_topk=1, routed_scale=2.5)
    idx_o = torch.empty((S, K), dtype=torch.int32, device=dev)
    w_o = torch.empty((S, K), dtype=torch.float32, device=dev)
    out, ws = b.moe_layer(rp, dev_bank(bank, dev), dev_bank(shared, dev), to_dev(x, dev),
                          idx_out=idx_o, w_out=w_o)
    torch.cuda.synchronize()
    r = orc.router(Wr, bias, x, K, 1, 2.5)
    np.testing.assert_array_equal(idx_o.cpu().numpy(), r["idx"])
    np.testing.assert_allclose(w_o.cpu().numpy(), r["w"], rtol=1e-6)
    toks = np.sort(g.choice(S, 16, replace=False))
    ref = orc.moe(bank, shared, x[toks], r["idx"][toks], r["w"][toks])
    assert_within(out.cpu().numpy()[toks], ref["out"], ref["mag"], REL, what="layer64")


@pytest.mark.parametrize("topp", [0.3, 0.85])
def test_layer_decode_64_tokens_topp(dev, orc, glm_bank, topp):
    """The 64-token layer (router N(0,0.02), bias U[-0.1,0.1], 256 int4
    experts of 6144 x 2048, shared expert) with top-p routing: ids and keff
    exact on all 64 tokens, out on 16 sampled tokens against the oracle's
    block on its own truncated routing."""
    bank, shared = glm_bank
    g = synth.rng(3003, int(topp * 100))
    S, K, E, D = 64, 8, 256, 6144
    Wr, bias = synth.router_weights(g, E, D)
    x = synth.activations(g, S, D)
    announce("moe layer 64 tokens topp", topp)
    out, idx, w, _ = run_layer_topp(dev, dev_bank(bank, dev), dev_bank(shared, dev), Wr, bias, x, K, topp)
    r = check_topp_routing(orc, Wr, bias, x, K, topp, idx, w, f"topp{topp} layer64")
    toks = np.sort(g.choice(S, 16, replace=False))
    ref = orc.moe(bank, shared, x[toks], r["idx"][toks], r["w"][toks])
    assert_within(out[toks], ref["out"], ref["mag"], REL, what=f"layer64 topp{topp}")
