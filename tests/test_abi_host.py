"""Host-only checks of the C ABI: the library loads, exports every function
include/coli.h declares, and rejects bad arguments before touching a device
(no compute call is made, so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli.h")


@pytest.fixture(scope="module")
def L():
    from weight_streaming_gemv_qgemv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from weight_streaming_gemv_qgemv_amd import build
        build.build()
    return binding.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(coli_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("coli_qgemv", "coli_moe_gemv", "coli_moe_layer", "coli_router",
              "coli_check_device_flags", "coli_strerror", "coli_moe_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_binding_covers_exports():
    from weight_streaming_gemv_qgemv_amd import binding
    assert set(binding.EXPORTS) == set(_declared())


def test_row_bytes_and_strerror(L):
    from weight_streaming_gemv_qgemv_amd import binding as b
    assert [b.row_bytes(f, 7) for f in (0, 1, 2, 3)] == [28, 7, 4, 2]
    assert b.row_bytes(2, 6144) == 3072 and b.row_bytes(3, 6144) == 1536
    assert b.row_bytes(9, 4) == -1 and b.row_bytes(2, -1) == -1
    for s in range(-8, 1):
        assert b.strerror(s)
    assert L.coli_version() >= 10000


FAKE = 0x10000  # a 16-byte aligned non-null pointer value; never dereferenced


def test_qgemv_rejects_before_launch(L):
    from weight_streaming_gemv_qgemv_amd import binding as b
    q = b.qgemv_raw
    assert q(4, FAKE, FAKE, FAKE, FAKE, 1, 8, 8) == b.EFMT
    assert q(-1, FAKE, FAKE, FAKE, FAKE, 1, 8, 8) == b.EFMT
    assert q(2, FAKE, FAKE, FAKE, FAKE, -1, 8, 8) == b.ESHAPE
    assert q(2, FAKE, FAKE, FAKE, FAKE, 1, -8, 8) == b.ESHAPE
    assert q(2, FAKE, FAKE, FAKE, None, 1, 8, 8) == b.EINVAL
    assert q(2, None, FAKE, FAKE, FAKE, 1, 8, 8) == b.EINVAL
    assert q(2, FAKE, None, FAKE, FAKE, 1, 8, 8) == b.EINVAL      # int formats need scales
    assert q(2, FAKE + 1, FAKE, FAKE, FAKE, 1, 8, 8) == b.EALIGN
    assert q(2, FAKE, FAKE, FAKE + 2, FAKE, 1, 8, 8) == b.EALIGN
    # empty batches are valid no-ops (nothing is launched)
    assert q(2, FAKE, FAKE, FAKE, FAKE, 0, 8, 8) == b.OK
    assert q(2, FAKE, FAKE, FAKE, FAKE, 3, 8, 0) == b.OK
    # overflow of S*O*4
    assert q(0, FAKE, FAKE, FAKE, FAKE, 2**31 - 1, 2**31 - 1, 2**31 - 1) == b.ESHAPE


def test_router_rejects_before_launch(L):
    from weight_streaming_gemv_qgemv_amd import binding as b
    r = L.coli_router
    ws = b.router_workspace_bytes(4, 16, 64)
    assert ws > 0
    args = dict(Wr=FAKE, bias=FAKE, x=FAKE, S=4, E=16, D=64, K=4, norm=1, rs=2.5, topp=0.0,
                idx=FAKE, w=FAKE, keff=None, sig=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return r(a["Wr"], a["bias"], a["x"], a["S"], a["E"], a["D"], a["K"], a["norm"], a["rs"],
                 a["topp"], a["idx"], a["w"], a["keff"], a["sig"], a["ws"], a["wsb"], None)

    assert call(K=17) == b.ERANGE
    assert call(K=0) == b.ERANGE
    assert call(E=2000, K=4) == b.ERANGE
    assert call(K=65, E=100) == b.ERANGE
    assert call(sig=None) == b.EINVAL
    assert call(norm=2) == b.EINVAL
    assert call(ws=None) == b.EWORKSPACE
    assert call(wsb=ws - 8) == b.EWORKSPACE
    assert call(x=FAKE + 2) == b.EALIGN
    assert call(S=0) == b.OK


def test_moe_rejects_before_launch(L):
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 64, 32, 4, 2
    ex = b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = b.moe_workspace_bytes(S, K, E, D, F, 0, 0)
    assert need > 0

    def call(ex=ex, x=FAKE, S=S, K=K, idx=FAKE, w=FAKE, out=FAKE, prec=0, ws=FAKE, wsb=need):
        return L.coli_moe_gemv(C.byref(ex), x, S, K, idx, w, out, prec, ws, wsb, None)

    assert call(wsb=need - 1) == b.EWORKSPACE
    assert call(ws=None) == b.EWORKSPACE
    assert call(ws=FAKE + 16) == b.EALIGN
    assert call(K=65) == b.ERANGE
    assert call(prec=7) == b.EINVAL
    assert call(idx=None) == b.EINVAL
    assert call(S=0) == b.OK
    bad = b.Experts(0, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)   # f32 experts unsupported
    assert call(ex=bad) == b.EFMT
    big = b.Experts(2, 2048, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ex=big) == b.ERANGE
    nul = b.Experts(2, E, D, F, FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert call(ex=nul) == b.EINVAL
    # layer: routing given as only one of the pair
    rp = b.RouterParams(FAKE, FAKE, K, 1, 2.5, 0.0)
    assert L.coli_moe_layer(C.byref(rp), C.byref(ex), None, FAKE, S, FAKE, None, FAKE, None, None,
                            0, FAKE, need, None) == b.EINVAL


def test_moe_refuses_sizes_past_32bit_offsets(L):
    """The expert kernels use 32-bit byte offsets into one weight matrix and
    one activation table; sizes past 2^32 - 4096 bytes are refused on the
    host (COLI_ERANGE) instead of wrapping on the device."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, K = 256, 6144, 2048, 8
    ex = b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    sh = b.Mlp(2, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    rp = b.RouterParams(FAKE, FAKE, K, 1, 2.5, 0.0)

    def layer(S, shared, prec):
        # one byte short of the workspace: a size that passes the range check
        # stops at the workspace check, so nothing is ever launched
        need = b.moe_workspace_bytes(S, K, E, D, F, F if shared else 0, prec)
        return L.coli_moe_layer(C.byref(rp), C.byref(ex), C.byref(sh) if shared else None, FAKE, S,
                                FAKE, FAKE, FAKE, None, None, prec, FAKE, need - 1, None)

    # fp32 precision: (9 S rows) x 4 x 2048 bytes of SwiGLU table
    assert layer(58255, True, 0) == b.ERANGE
    assert layer(58254, True, 0) == b.EWORKSPACE
    assert layer(65536, False, 0) == b.ERANGE        # 8 S rows
    assert layer(65535, False, 0) == b.EWORKSPACE
    # bf16 precision: 2 bytes per element, twice the tokens
    assert layer(2 * 58255, True, 1) == b.ERANGE
    assert layer(2 * 58254, True, 1) == b.EWORKSPACE
    # one expert matrix of 2^32 bytes (int4, D = 2^20, F = 8192)
    big = b.Experts(2, 4, 1 << 20, 8192, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = b.moe_workspace_bytes(1, 2, 4, 1 << 20, 8192, 0, 0)
    assert L.coli_moe_gemv(C.byref(big), FAKE, 1, 2, FAKE, FAKE, FAKE, 0, FAKE, need - 1, None) == b.ERANGE


def test_noalloc_layer_refuses_before_any_device_call(L):
    """coli_moe_layer_noalloc: a workspace past its static scratch is refused
    (COLI_ERANGE) before the device is touched, and NULL structs are EINVAL."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    ex = b.Experts(2, 256, 6144, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    rp = b.RouterParams(FAKE, FAKE, 8, 1, 2.5, 0.0)
    f = L.coli_moe_layer_noalloc
    assert f(C.byref(rp), C.byref(ex), None, FAKE, 300, None, None, FAKE, None, None, 0, None) == b.ERANGE
    assert f(None, C.byref(ex), None, FAKE, 4, None, None, FAKE, None, None, 0, None) == b.EINVAL
    assert f(C.byref(rp), None, None, FAKE, 4, None, None, FAKE, None, None, 0, None) == b.EINVAL
    assert f(C.byref(rp), C.byref(ex), None, FAKE, 0, None, None, FAKE, None, None, 0, None) == b.OK


def test_tiled_layout_host_checks(L):
    """coli_tiled_bytes and the refusals of coli_pack_tiled / tiled experts
    (no device work)."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    assert b.tiled_bytes(2, 256, 2048, 6144) == 256 * 2048 * 3072      # whole units: no padding
    assert b.tiled_bytes(2, 1, 17, 96) == 2 * 1 * 1024                  # 2 row tiles x 1 segment
    assert b.tiled_bytes(1, 3, 40, 160) == 3 * 3 * 3 * 1024
    assert b.tiled_bytes(0, 1, 16, 64) == -1 and b.tiled_bytes(2, -1, 16, 64) == -1
    p = L.coli_pack_tiled
    assert p(0, FAKE, 1, 16, 64, FAKE, None) == b.EFMT
    assert p(2, FAKE, 1, 16, 40, FAKE, None) == b.EALIGN      # 20-byte rows
    assert p(2, FAKE + 4, 1, 16, 64, FAKE, None) == b.EALIGN
    assert p(2, None, 1, 16, 64, FAKE, None) == b.EINVAL
    assert p(2, FAKE, -1, 16, 64, FAKE, None) == b.ESHAPE
    assert p(2, FAKE, 0, 16, 64, FAKE, None) == b.OK            # nothing to pack
    E, D, F, S, K = 8, 64, 32, 4, 2
    need = b.moe_workspace_bytes(S, K, E, D, F, F, 0)

    def layer(ex, sh):
        return L.coli_moe_layer(C.byref(b.RouterParams(FAKE, FAKE, K, 1, 2.5, 0.0)), C.byref(ex),
                                C.byref(sh) if sh else None, FAKE, S, FAKE, FAKE, FAKE, None, None, 0,
                                FAKE, need - 1, None)
    rows = b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0)
    tiled = b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)
    sh_t = b.Mlp(2, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)
    sh_r = b.Mlp(2, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0)
    assert layer(tiled, sh_t) == b.EWORKSPACE                  # valid up to the workspace
    assert layer(tiled, sh_r) == b.EWORKSPACE                  # row-major shared: vector ALUs
    assert layer(rows, sh_t) == b.EINVAL                       # tiled shared needs tiled experts
    assert layer(b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 7), None) == b.EINVAL
    odd = b.Experts(2, E, 40, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)   # 20-byte rows of D
    assert layer(odd, None) == b.EALIGN


def test_workspace_layout_is_consistent(L):
    from weight_streaming_gemv_qgemv_amd import binding as b
    for (S, K, E, D, F, Fs) in [(1, 1, 1, 1, 1, 0), (64, 8, 256, 6144, 2048, 2048),
                                (2048, 8, 256, 6144, 2048, 2048), (5, 3, 24, 40, 24, 16)]:
        lay = b.moe_workspace_layout(S, K, E, D, F, Fs)
        assert lay["total"] == b.moe_workspace_bytes(S, K, E, D, F, Fs)
        regions = sorted((v, k) for k, v in lay.items()
                         if not k.endswith(("_ld", "_stride", "_max")) and k != "total")
        assert all(v % 256 == 0 for v, _ in regions)
        assert lay["h_ld"] == max(F, Fs)
        rows = S * K + (S if Fs else 0)
        assert lay["y"] + rows * D * 4 <= lay["total"]
        assert lay["h"] + rows * max(F, Fs) * 4 <= lay["y"]
        # bf16 precision: h's partial sums per grouped row, as many parts as
        # the grouped-scale prefill items need (KpF / 16), then the totals
        lb = b.moe_workspace_layout(S, K, E, D, F, Fs, b.PREC_BF16)
        kpf = -(-max(F, Fs) // 1024) * 1024
        ends = sorted(v for k, v in lb.items() if not k.endswith(("_ld", "_stride", "_max")) and v >= 0)
        nxt = min([v for v in ends if v > lb["hsum"]] + [lb["total"]])
        assert nxt - lb["hsum"] >= rows * (kpf // 16 + 1) * 4


def test_idot_precision_host_checks(L):
    """COLI_PREC_IDOT takes int8 / int4 experts in the tiled layout (and a
    shared expert of the same format, F and layout) only; the workspace
    regions hold the int8 tables, scales and sums of S tokens and of the
    grouped rows."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    E, D, F, S, K = 8, 64, 32, 4, 2

    def layer(ex, sh):
        # one byte short of the workspace this call needs: a call the checks
        # accept stops at COLI_EWORKSPACE, before any device work
        need = b.moe_workspace_bytes(S, K, E, ex.D, ex.F, sh.F if sh else 0, b.PREC_IDOT)
        assert need > 0
        return L.coli_moe_layer(C.byref(b.RouterParams(FAKE, FAKE, K, 1, 2.5, 0.0)), C.byref(ex),
                                C.byref(sh) if sh else None, FAKE, S, FAKE, FAKE, FAKE, None, None,
                                b.PREC_IDOT, FAKE, need - 1, None)
    tiled4 = b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)
    assert layer(tiled4, None) == b.EWORKSPACE                 # valid up to the workspace
    assert layer(b.Experts(1, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1), None) == b.EWORKSPACE
    assert layer(b.Experts(3, E, D, 2 * F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1), None) == b.EFMT  # int2
    assert layer(b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0), None) == b.EINVAL  # rows
    assert layer(tiled4, b.Mlp(2, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0)) == b.EINVAL  # rows shared
    assert layer(tiled4, b.Mlp(2, 2 * F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)) == b.EINVAL
    assert layer(tiled4, b.Mlp(2, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)) == b.EWORKSPACE
    wide = b.Experts(2, E, 16416, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)
    assert layer(wide, None) == b.ERANGE
    for Fs in (0, F):
        lay = b.moe_workspace_layout(S, K, E, D, F, Fs, b.PREC_IDOT)
        rows = S * K + (S if Fs else 0)
        kp = lambda n: (n + 1023) // 1024 * 1024
        assert lay["xsum"] - lay["xf"] >= S * kp(D)
        assert lay["hf"] - lay["xsum"] >= (5 * S + 3 * rows) * 4
        assert lay["hsum"] - lay["hf"] >= rows * kp(F)
        assert lay["work"] - lay["hsum"] >= rows * 7 * 4


def test_grouped_scale_host_checks(L):
    """Grouped-scale int4 experts: gs one of 32 .. 1024, fmt int4, the grouped
    tiled layout exactly when gs > 0, fp32 or bf16 precision (no integer
    dots), a tiled shared expert of the same gs; the packed scale sizes (no
    device work)."""
    from weight_streaming_gemv_qgemv_amd import binding as b
    assert b.grouped_scale_bytes(1, 16, 64, 32) == 1 * 1 * (1024 // 32) * 64
    assert b.grouped_scale_bytes(3, 17, 1025, 128) == 3 * 2 * (2048 // 128) * 64
    assert b.grouped_scale_bytes(256, 2048, 6144, 128) == 256 * 128 * 48 * 64
    for bad in (0, 16, 48, 2048):
        assert b.grouped_scale_bytes(1, 16, 64, bad) == -1
    ps = L.coli_pack_scales_grouped
    assert ps(FAKE, 1, 16, 64, 48, FAKE, None) == b.ERANGE
    assert ps(FAKE, 1, 16, 64, 32, FAKE + 4, None) == b.EALIGN
    assert ps(None, 1, 16, 64, 32, FAKE, None) == b.EINVAL
    assert ps(FAKE, 0, 16, 64, 32, FAKE, None) == b.OK
    pt = L.coli_pack_tiled_grouped
    assert pt(FAKE, 1, 16, 40, FAKE, None) == b.EALIGN          # 20-byte rows
    assert pt(None, 1, 16, 64, FAKE, None) == b.EINVAL
    assert pt(FAKE, 0, 16, 64, FAKE, None) == b.OK
    E, D, F, S, K = 8, 64, 64, 4, 2

    def layer(ex, sh, prec=b.PREC_FP32):
        need = b.moe_workspace_bytes(S, K, E, ex.D, ex.F, sh.F if sh else 0, prec)
        assert need > 0
        return L.coli_moe_layer(C.byref(b.RouterParams(FAKE, FAKE, K, 1, 2.5, 0.0)), C.byref(ex),
                                C.byref(sh) if sh else None, FAKE, S, FAKE, FAKE, FAKE, None, None,
                                prec, FAKE, need - 1, None)

    def ex(fmt=2, layout=2, gs=32):
        return b.Experts(fmt, E, D, F, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, layout, gs)

    def sh(layout=2, gs=32, Fs=F):
        return b.Mlp(2, Fs, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, layout, gs)
    assert layer(ex(), None) == b.EWORKSPACE                     # valid up to the workspace
    assert layer(ex(gs=1024), sh(gs=1024)) == b.EWORKSPACE
    assert layer(ex(), sh(layout=0, gs=0)) == b.EWORKSPACE       # row-major shared, per-row scales
    assert layer(ex(gs=48), None) == b.ERANGE
    assert layer(ex(layout=1), None) == b.EINVAL                 # grouped scales need layout 2
    assert layer(ex(gs=0), None) == b.EINVAL                     # layout 2 needs grouped scales
    assert layer(ex(fmt=1), None) == b.EFMT                      # int4 only
    assert layer(ex(), None, b.PREC_BF16) == b.EWORKSPACE         # the bf16 prefill kernels take them too
    assert layer(ex(), None, b.PREC_IDOT) == b.EFMT
    assert layer(ex(), sh(gs=64)) == b.EINVAL                    # shared gs differs
    assert layer(ex(), sh(Fs=2 * F)) == b.EINVAL
    assert layer(b.Experts(2, E, D, F, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 2, 32), None) == b.EALIGN
