"""GPU parity of the integer-dot expert path (COLI_PREC_IDOT) against the
oracle's integer-dot MoE block (oracle.moe_idot).

Per token the layer quantises x to int8 once; every expert product is an
exact int32 dot with the pages' fp32 epilogue.  The checks, stage by stage:
  * h (gate/up, SwiGLU) against the oracle's h: the integer dots and their
    epilogue are the same, so the two differ only by the platforms' expf
    inside silu, whose relative error grows with its argument: within
    2^-21 (1 + |g|) relative, g the gate value (a dot off by one unit moves
    h by about 1/|dot|, 1e-4 to 1e-5 here);
  * y (down) bit for bit against the oracle's down products taken on the
    GPU's own h rows (oracle.moe_idot(..., h_in=h_gpu));
  * out against the fp64 weighted sum of those y (the combine's fp32
    rounding: 2e-6 of sum |w y|)."""
import numpy as np
import pytest

from gpu_helpers import announce, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
PREC_IDOT = 2


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _dev_bank(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def run_idot_layer(dev, bank, shared, x, idx, w):
    """The layer on tiled copies of the banks; returns out and the per-pair
    h and y rows (pair p = s K + kk, shared rows at S K + s) read from the
    workspace."""
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    S, K = idx.shape
    E, D, F = bank["E"], bank["D"], bank["F"]
    td = b.tile_mlps(_dev_bank(bank, dev))
    tsd = b.tile_mlps(_dev_bank(shared, dev), D) if shared is not None else None
    out, ws = b.moe_layer(None, td, tsd, to_dev(x, dev), pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev),
                          prec=PREC_IDOT)
    torch.cuda.synchronize()
    L = b.moe_workspace_layout(S, K, E, D, F, F if shared is not None else 0, PREC_IDOT)
    raw = ws.cpu().numpy()
    P = S * K
    rows = P + (S if shared is not None else 0)
    pair_row = raw[L["pair_row"]:L["pair_row"] + 4 * P].view(np.int32)
    h_all = raw[L["h"]:L["h"] + 4 * rows * L["h_ld"]].view(np.float32).reshape(rows, L["h_ld"])[:, :F]
    y_all = raw[L["y"]:L["y"] + 4 * rows * D].view(np.float32).reshape(rows, D)
    gr = np.concatenate([pair_row, P + np.arange(rows - P)]).astype(np.int64)
    valid = gr >= 0
    h = np.zeros((rows, F), np.float32)
    y = np.zeros((rows, D), np.float32)
    h[valid] = h_all[gr[valid]]
    y[valid] = y_all[gr[valid]]
    return out.cpu().numpy(), h, y, valid


def check_stages(orc, bank, shared, x, idx, w, out, h, y, valid, what):
    ref = orc.moe_idot(bank, shared, x, idx, w)
    tol = 2.0 ** -21 * (1.0 + np.abs(ref["g"][valid].astype(np.float64))) * np.abs(ref["h"][valid]) + 1e-35
    dh = np.abs(h[valid].astype(np.float64) - ref["h"][valid])
    assert np.all(dh <= tol), (what + " h", int((dh > tol).sum()), float((dh / tol).max()))
    ref2 = orc.moe_idot(bank, shared, x, idx, w, h_in=h)
    np.testing.assert_array_equal(y[valid].view(np.uint32), ref2["y"][valid].view(np.uint32),
                                  err_msg=what + " y bits")
    S, K = idx.shape
    wab = np.abs(w.astype(np.float64))
    mag = np.zeros_like(ref2["out"])
    for kk in range(K):
        p = np.arange(S) * K + kk
        ok = idx[:, kk] >= 0
        mag[ok] += wab[ok, kk][:, None] * np.abs(ref2["y"][p[ok]].astype(np.float64))
    if shared is not None:
        mag += np.abs(ref2["y"][S * K:].astype(np.float64))
    assert np.all(np.abs(out - ref2["out"]) <= 2e-6 * mag + 1e-30), what + " out"


@pytest.mark.parametrize("fmt", [1, 2])
def test_idot_layer_small(dev, orc, fmt):
    E, D, F, S, K = 16, 1024, 512, 300, 4
    bank = synth.expert_bank(90 + fmt, fmt, E, D, F)
    shared = synth.shared_mlp(90 + fmt, fmt, D, F)
    g = synth.rng(91, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    assert np.bincount(idx.ravel(), minlength=E).max() > 64   # multi-pass experts
    announce("idot layer small", fmt)
    out, h, y, valid = run_idot_layer(dev, bank, shared, x, idx, w)
    check_stages(orc, bank, shared, x, idx, w, out, h, y, valid, f"idot small fmt{fmt}")


def test_idot_layer_ragged_no_shared(dev, orc):
    """Empty slots, a width that is not a multiple of the k-block (D = 1056,
    F = 160: zero-padded int8 rows), no shared expert."""
    fmt, E, D, F, S, K = 2, 8, 1056, 160, 70, 3
    bank = synth.expert_bank(95, fmt, E, D, F)
    g = synth.rng(96)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[::7, 1] = -1
    announce("idot layer ragged")
    out, h, y, valid = run_idot_layer(dev, bank, None, x, idx, w)
    check_stages(orc, bank, None, x, idx, w, out, h, y, valid, "idot ragged")


def test_idot_prefill_2048(dev, orc, glm_bank):
    """The prefill workload on the integer-dot path: 2048 tokens, 256 int4
    experts + shared, Zipf(1.1) routing; 24 sampled tokens' h, y and out
    against the oracle."""
    bank, shared = glm_bank
    S, K, E, D = 2048, 8, 256, 6144
    g = synth.rng(5600)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    announce("idot prefill 2048")
    out, h, y, valid = run_idot_layer(dev, bank, shared, x, idx, w)
    toks = np.sort(g.choice(S, 24, replace=False))
    pairs = (toks[:, None] * K + np.arange(K)[None, :]).ravel()
    sel = np.concatenate([pairs, S * K + toks])
    check_stages(orc, bank, shared, x[toks], idx[toks], w[toks], out[toks], h[sel], y[sel], valid[sel],
                 "idot prefill2048")
