"""GPU parity of the prefill precision (COLI_PREC_BF16) against the oracle.

Activations (x, and h for the down product) are rounded once to bf16 for
the matrix cores; int weights become exact bf16 codes; accumulation is
fp32.  Bar, elementwise on the layer output:
    |out - ref| <= 2e-2 * M_out + 1e-6,
with M_out the oracle's fp64 chain magnitude (sum_k |w_k| |sd[o]| sum_j
|vd(o,j) h_j| plus the shared expert's term).  The per-row relative L2
error is reported beside it.  Routing is Zipf(1.1)-skewed, so some experts
carry many rows (several 64-row passes)."""
import numpy as np
import pytest

from gpu_helpers import announce, assert_within, need_gpu, to_dev
from weight_streaming_gemv_qgemv_amd import synth

pytestmark = pytest.mark.gpu
REL = 2e-2
PREC_BF16 = 1


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def dev_bank(bank, dev):
    out = dict(bank)
    for k in ("wg", "wu", "wd", "sg", "su", "sd"):
        out[k] = to_dev(bank[k], dev)
    return out


def run_layer(dev, bank, shared, x, idx, w, prec):
    import torch
    from weight_streaming_gemv_qgemv_amd import binding as b
    out, ws = b.moe_layer(None, dev_bank(bank, dev), dev_bank(shared, dev) if shared else None,
                          to_dev(x, dev), pre_idx=to_dev(idx, dev), pre_w=to_dev(w, dev),
                          prec=prec)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def rel_l2(got, ref):
    d = np.linalg.norm(np.asarray(got, np.float64) - ref, axis=1)
    return float((d / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)).max())


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_prefill_bf16_small(dev, orc, fmt):
    E, D, F, S, K = 16, 1024, 512, 300, 4
    bank = synth.expert_bank(60 + fmt, fmt, E, D, F)
    shared = synth.shared_mlp(60 + fmt, fmt, D, F)
    g = synth.rng(61, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    assert np.bincount(idx.ravel(), minlength=E).max() > 32   # multi-pass experts
    announce("prefill bf16 small", fmt)
    out, _ = run_layer(dev, bank, shared, x, idx, w, PREC_BF16)
    ref = orc.moe(bank, shared, x, idx, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what=f"prefill fmt{fmt}")
    # bf16 rounding is visible (not the fp32 path) but small
    assert rel_l2(out, ref["out"]) < 2e-2


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_prefill_bf16_short_rows(dev, orc, fmt):
    """Rows of whole 16-byte segments shorter than 64 bytes (D=64, F=32)."""
    E, D, F, S, K = 8, 64, 32, 90, 3
    bank = synth.expert_bank(65 + fmt, fmt, E, D, F)
    shared = synth.shared_mlp(65 + fmt, fmt, D, F)
    g = synth.rng(66, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    announce("prefill bf16 short rows", fmt)
    out, _ = run_layer(dev, bank, shared, x, idx, w, PREC_BF16)
    ref = orc.moe(bank, shared, x, idx, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what=f"prefill short fmt{fmt}")


@pytest.mark.parametrize("fmt", [1, 2])
def test_prefill_bf16_no_shared_expert(dev, orc, fmt):
    """The matrix-core prefill path without a shared expert (the workspace
    then has no shared rows: the grouped-row tables are sized P = S K) and
    with empty slots."""
    E, D, F, S, K = 12, 1024, 512, 200, 4
    bank = synth.expert_bank(75 + fmt, fmt, E, D, F)
    g = synth.rng(76, fmt)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    idx[::5, 2] = -1
    announce("prefill bf16 no shared", fmt)
    out, _ = run_layer(dev, bank, None, x, idx, w, PREC_BF16)
    ref = orc.moe(bank, None, x, idx, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], REL, what=f"prefill no shared fmt{fmt}")


def test_prefill_bf16_unaligned_rows_take_fp32(dev, orc):
    """Rows that are not whole 16-byte segments take the vector-ALU kernels,
    which compute in fp32 under either precision."""
    E, D, F, S, K = 8, 1000, 200, 40, 3
    bank = synth.expert_bank(70, 2, E, D, F)
    g = synth.rng(71)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    announce("prefill bf16 unaligned")
    out, _ = run_layer(dev, bank, None, x, idx, w, PREC_BF16)
    ref = orc.moe(bank, None, x, idx, w.astype(np.float64))
    assert_within(out, ref["out"], ref["mag"], 1e-4, what="unaligned")


def test_prefill_2048_tokens(dev, orc, glm_bank):
    """The prefill workload: 2048 tokens through 256 int4 experts + shared,
    Zipf(1.1) routing, bf16 matrix cores; 24 sampled tokens against the
    oracle."""
    bank, shared = glm_bank
    g = synth.rng(5000)
    S, K, E, D = 2048, 8, 256, 6144
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert counts.max() > 1000 and (counts > 0).sum() > 200
    announce("prefill 2048 tokens")
    out, _ = run_layer(dev, bank, shared, x, idx, w, PREC_BF16)
    assert np.all(np.isfinite(out))
    toks = np.sort(g.choice(S, 24, replace=False))
    ref = orc.moe(bank, shared, x[toks], idx[toks], w[toks].astype(np.float64))
    assert_within(out[toks], ref["out"], ref["mag"], REL, what="prefill2048")
    assert rel_l2(out[toks], ref["out"]) < 2e-2


def expected_work(counts, extra, tpp=64):
    """The prefill work list: entry g | pass << 11 for each tpp-row pass of
    each group (experts, then the shared expert's group), sorted by the
    pass's live 16-row tiles (4, 3, 2, 1), group and pass order inside a
    class; ends = [total, end of class 0, .., end of class 3]."""
    classes = [[] for _ in range(tpp // 16)]
    for g, c in enumerate(list(counts) + [extra]):
        for p in range(-(-int(c) // tpp)):
            live = min(tpp, int(c) - p * tpp)
            classes[tpp // 16 - -(-live // 16)].append(g | (p << 11))
    ends = np.cumsum([len(c) for c in classes]).tolist()
    return [e for c in classes for e in c], [ends[-1]] + ends


@pytest.mark.parametrize("S,K,E", [(90, 3, 8), (300, 4, 16), (1000, 8, 64)])
def test_prefill_work_list_classes(dev, S, K, E):
    """The grouping's prefill work list, from both grouping paths (one
    launch for at most 1024 slots, chunked beyond), exactly."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    D, F = 256, 128
    bank = synth.expert_bank(80, 2, E, D, F)
    shared = synth.shared_mlp(80, 2, D, F)
    g = synth.rng(81, S)
    x = synth.activations(g, S, D)
    idx, w = synth.routing_zipf(g, S, K, E)
    announce("prefill work list", S, K, E)
    _, ws = run_layer(dev, bank, shared, x, idx, w, PREC_BF16)
    L = b.moe_workspace_layout(S, K, E, D, F, F, PREC_BF16)
    raw = ws.cpu().numpy()
    ends = raw[L["n_work"]:L["n_work"] + 20].view(np.int32)
    want, want_ends = expected_work(np.bincount(idx.ravel(), minlength=E), S)
    assert ends[:5].tolist() == want_ends
    got = raw[L["work"]:L["work"] + 4 * len(want)].view(np.int32)
    assert got.tolist() == want
