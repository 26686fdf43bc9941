"""ctypes binding of libcoli.so (include/coli.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and every step of the computation runs in the
library's HIP kernels.  There is no fallback: if libcoli.so is missing or a
call fails, this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoli.so")

F32, I8, I4, I2 = 0, 1, 2, 3
PREC_FP32, PREC_BF16, PREC_IDOT = 0, 1, 2
LAYOUT_ROWS, LAYOUT_TILED, LAYOUT_TILED_GROUPED = 0, 1, 2
OK, EINVAL, ESHAPE, EFMT, EALIGN, ERANGE, EWORKSPACE, EDEVICE, EIDX = 0, -1, -2, -3, -4, -5, -6, -7, -8


class ColiError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


class Experts(C.Structure):
    _fields_ = [("fmt", C.c_int), ("E", C.c_int), ("D", C.c_int), ("F", C.c_int),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p),
                ("layout", C.c_int), ("gs", C.c_int)]


class Mlp(C.Structure):
    _fields_ = [("fmt", C.c_int), ("F", C.c_int),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p),
                ("layout", C.c_int), ("gs", C.c_int)]


class RouterParams(C.Structure):
    _fields_ = [("w", C.c_void_p), ("bias", C.c_void_p), ("K", C.c_int),
                ("norm_topk", C.c_int), ("routed_scale", C.c_float), ("topp", C.c_float)]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("flags", "sig", "idx", "w", "offsets", "counts",
                                          "row_pair", "pair_row", "h", "y", "router_part",
                                          "xf", "xsum", "hf", "hsum", "work", "n_work", "xn", "gpart",
                                          "n_pass_max", "xf_stride", "hf_stride", "h_ld", "total")]


EXPORTS = ["coli_row_bytes", "coli_qgemv", "coli_router", "coli_router_workspace_bytes",
           "coli_moe_workspace_bytes", "coli_moe_workspace_layout", "coli_moe_gemv",
           "coli_moe_layer", "coli_moe_layer_tail", "coli_qgemv_idot", "coli_qgemv_grouped",
           "coli_qgemv_idot_workspace_bytes", "coli_check_device_flags", "coli_strerror", "coli_version",
           "coli_stage_timing", "coli_stage_times", "coli_stage_name", "coli_moe_layer_noalloc",
           "coli_tiled_bytes", "coli_pack_tiled", "coli_pack_tiled_grouped", "coli_grouped_scale_bytes",
           "coli_pack_scales_grouped"]
NSTAGES = 8

_lib = None


def lib():
    """Load libcoli.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m weight_streaming_gemv_qgemv_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
        L.coli_row_bytes.restype = i64
        L.coli_row_bytes.argtypes = [i32, i64]
        L.coli_qgemv.restype = i32
        L.coli_qgemv.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, vp]
        L.coli_router.restype = i32
        L.coli_router.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, vp, vp, vp, vp,
                                  vp, sz, vp]
        L.coli_router_workspace_bytes.restype = sz
        L.coli_router_workspace_bytes.argtypes = [i32, i32, i32]
        L.coli_moe_workspace_bytes.restype = sz
        L.coli_moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.coli_moe_workspace_layout.restype = i32
        L.coli_moe_workspace_layout.argtypes = [i32, i32, i32, i32, i32, i32, i32, C.POINTER(WsLayout)]
        L.coli_moe_gemv.restype = i32
        L.coli_moe_gemv.argtypes = [C.POINTER(Experts), vp, i32, i32, vp, vp, vp, i32, vp, sz, vp]
        L.coli_moe_layer.restype = i32
        L.coli_moe_layer.argtypes = [C.POINTER(RouterParams), C.POINTER(Experts), C.POINTER(Mlp),
                                     vp, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.coli_tiled_bytes.restype = i64
        L.coli_tiled_bytes.argtypes = [i32, i64, i32, i32]
        L.coli_pack_tiled.restype = i32
        L.coli_pack_tiled.argtypes = [i32, vp, i64, i32, i32, vp, vp]
        L.coli_pack_tiled_grouped.restype = i32
        L.coli_pack_tiled_grouped.argtypes = [vp, i64, i32, i32, vp, vp]
        L.coli_grouped_scale_bytes.restype = i64
        L.coli_grouped_scale_bytes.argtypes = [i64, i32, i32, i32]
        L.coli_pack_scales_grouped.restype = i32
        L.coli_pack_scales_grouped.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        L.coli_moe_layer_noalloc.restype = i32
        L.coli_moe_layer_noalloc.argtypes = [C.POINTER(RouterParams), C.POINTER(Experts), C.POINTER(Mlp),
                                             vp, i32, vp, vp, vp, vp, vp, i32, vp]
        L.coli_qgemv_grouped.restype = i32
        L.coli_qgemv_grouped.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, vp]
        L.coli_qgemv_idot_workspace_bytes.restype = sz
        L.coli_qgemv_idot_workspace_bytes.argtypes = [i32, i32]
        L.coli_qgemv_idot.restype = i32
        L.coli_qgemv_idot.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, vp, sz, vp]
        L.coli_moe_layer_tail.restype = i32
        L.coli_moe_layer_tail.argtypes = [C.POINTER(RouterParams), C.POINTER(Experts), C.POINTER(Mlp),
                                          vp, vp, C.c_float, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.coli_check_device_flags.restype = i32
        L.coli_check_device_flags.argtypes = [vp, vp, C.POINTER(C.c_uint32)]
        L.coli_strerror.restype = C.c_char_p
        L.coli_strerror.argtypes = [i32]
        L.coli_version.restype = i32
        L.coli_version.argtypes = []
        L.coli_stage_timing.restype = i32
        L.coli_stage_timing.argtypes = [i32]
        L.coli_stage_times.restype = i32
        L.coli_stage_times.argtypes = [vp, vp, i32]
        L.coli_stage_name.restype = C.c_char_p
        L.coli_stage_name.argtypes = [i32]
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().coli_strerror(status).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc: int, what: str):
    if rc != OK:
        raise ColiError(rc, what)


def _nbytes(t) -> int | None:
    """Bytes a tensor argument holds (None for a raw pointer or None)."""
    if t is None or isinstance(t, int):
        return None
    return t.numel() * t.element_size()


def _need(t, nbytes: int, what: str):
    """The library takes raw pointers and cannot see allocation sizes: a
    tensor smaller than the call reads or writes is refused here, before
    anything runs on the device."""
    have = _nbytes(t)
    if have is not None and have < nbytes:
        raise ColiError(ESHAPE, f"{what}: tensor holds {have} bytes, the call needs {nbytes}")


def row_bytes(fmt: int, I: int) -> int:
    return int(lib().coli_row_bytes(fmt, I))


# ------------------------------------------------------------------ qgemv
def qgemv(fmt: int, W: torch.Tensor, scale, x: torch.Tensor, y: torch.Tensor | None = None,
          O: int | None = None, stream=None) -> torch.Tensor:
    """y[s,o] = scale[o] * sum_i v(o,i) x[s,i]; W [O, row_bytes] uint8 (or f32 [O, I])."""
    S, I = x.shape
    if O is None:
        if W.dim() != 2:
            raise ColiError(EINVAL, "qgemv: pass O for a weight tensor that is not [O, row bytes]")
        O = W.shape[0]
    if y is None:
        y = torch.empty((S, O), dtype=torch.float32, device=x.device)
    _need(W, O * row_bytes(fmt, I), "qgemv W")
    _need(scale, 4 * O, "qgemv scale")
    _need(y, 4 * S * O, "qgemv y")
    rc = lib().coli_qgemv(fmt, _ptr(W), _ptr(scale), _ptr(x), _ptr(y), S, I, O, _stream(stream))
    _check(rc, "coli_qgemv")
    return y


def qgemv_grouped(W: torch.Tensor, scale: torch.Tensor, gs: int, x: torch.Tensor,
                  y: torch.Tensor | None = None, O: int | None = None, stream=None) -> torch.Tensor:
    """Grouped-scale int4: scale [O, ceil(I/gs)], one per gs elements along I."""
    S, I = x.shape
    if O is None:
        if W.dim() != 2:
            raise ColiError(EINVAL, "qgemv_grouped: pass O for a weight tensor that is not [O, row bytes]")
        O = W.shape[0]
    if y is None:
        y = torch.empty((S, O), dtype=torch.float32, device=x.device)
    _need(W, O * row_bytes(I4, I), "qgemv_grouped W")
    _need(scale, 4 * O * (-(-I // max(int(gs), 1))), "qgemv_grouped scale")
    _need(y, 4 * S * O, "qgemv_grouped y")
    rc = lib().coli_qgemv_grouped(_ptr(W), _ptr(scale), int(gs), _ptr(x), _ptr(y), S, I, O, _stream(stream))
    _check(rc, "coli_qgemv_grouped")
    return y


def qgemv_idot_workspace_bytes(S: int, I: int) -> int:
    return int(lib().coli_qgemv_idot_workspace_bytes(S, I))


def qgemv_idot(fmt: int, W: torch.Tensor, scale, x: torch.Tensor, y: torch.Tensor | None = None,
               O: int | None = None, ws=None, stream=None):
    """Integer-dot qgemv (int8 / int4): x quantised to int8 per row by absmax/127."""
    S, I = x.shape
    if O is None:
        if W.dim() != 2:
            raise ColiError(EINVAL, "qgemv_idot: pass O for a weight tensor that is not [O, row bytes]")
        O = W.shape[0]
    if y is None:
        y = torch.empty((S, O), dtype=torch.float32, device=x.device)
    _need(W, O * row_bytes(fmt, I), "qgemv_idot W")
    _need(scale, 4 * O, "qgemv_idot scale")
    _need(y, 4 * S * O, "qgemv_idot y")
    if ws is None:
        ws = alloc_workspace(max(qgemv_idot_workspace_bytes(S, I), 256), x.device)
    rc = lib().coli_qgemv_idot(fmt, _ptr(W), _ptr(scale), _ptr(x), _ptr(y), S, I, O, _ptr(ws), ws.numel(),
                               _stream(stream))
    _check(rc, "coli_qgemv_idot")
    return y, ws


def qgemv_raw(fmt, W, scale, x, y, S, I, O, stream=0) -> int:
    """Direct call with raw pointers / sizes; returns the status code."""
    return int(lib().coli_qgemv(fmt, W, scale, x, y, S, I, O, stream))


# ------------------------------------------------------------------ router
def router_workspace_bytes(S: int, E: int, D: int) -> int:
    return int(lib().coli_router_workspace_bytes(S, E, D))


def router(Wr, bias, x, K: int, norm_topk: int = 1, routed_scale: float = 2.5, topp: float = 0.0,
           ws: torch.Tensor | None = None, stream=None):
    S, D = x.shape
    E = Wr.shape[0]
    dev = x.device
    idx = torch.empty((S, K), dtype=torch.int32, device=dev)
    w = torch.empty((S, K), dtype=torch.float32, device=dev)
    keff = torch.empty((S,), dtype=torch.int32, device=dev)
    sig = torch.empty((S, E), dtype=torch.float32, device=dev)
    nb = router_workspace_bytes(S, E, D)
    if ws is None:
        ws = torch.empty((max(nb, 256),), dtype=torch.uint8, device=dev)
    rc = lib().coli_router(_ptr(Wr), _ptr(bias), _ptr(x), S, E, D, K, norm_topk, routed_scale,
                           topp, _ptr(idx), _ptr(w), _ptr(keff), _ptr(sig), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check(rc, "coli_router")
    return dict(idx=idx, w=w, keff=keff, sig=sig)


# ------------------------------------------------------------------ MoE
def _check_mlp_sizes(d: dict, n: int, D: int, F: int, what: str):
    """Weight and scale tensors of n stacked experts of width D x F hold at
    least the bytes their layout needs."""
    fmt, lay, gs = d["fmt"], int(d.get("layout", LAYOUT_ROWS)), int(d.get("gs", 0))
    if lay in (LAYOUT_TILED, LAYOUT_TILED_GROUPED):
        gu, dn = tiled_bytes(fmt, n, F, D), tiled_bytes(fmt, n, D, F)
    else:
        gu, dn = n * F * row_bytes(fmt, D), n * D * row_bytes(fmt, F)
    _need(d["wg"], gu, what + " w_gate")
    _need(d["wu"], gu, what + " w_up")
    _need(d["wd"], dn, what + " w_down")
    if gs and lay == LAYOUT_TILED_GROUPED:
        sgu, sdn = grouped_scale_bytes(n, F, D, gs), grouped_scale_bytes(n, D, F, gs)
        if sgu < 0 or sdn < 0:
            raise ColiError(ERANGE, what + " gs")
    else:
        sgu, sdn = 4 * n * F, 4 * n * D
    _need(d["sg"], sgu, what + " s_gate")
    _need(d["su"], sgu, what + " s_up")
    _need(d["sd"], sdn, what + " s_down")


def experts_struct(ex: dict) -> Experts:
    _check_mlp_sizes(ex, ex["E"], ex["D"], ex["F"], "experts")
    return Experts(ex["fmt"], ex["E"], ex["D"], ex["F"], _ptr(ex["wg"]), _ptr(ex["wu"]),
                   _ptr(ex["wd"]), _ptr(ex["sg"]), _ptr(ex["su"]), _ptr(ex["sd"]),
                   int(ex.get("layout", LAYOUT_ROWS)), int(ex.get("gs", 0)))


def mlp_struct(sh: dict, D: int | None = None) -> Mlp:
    if D is not None:
        _check_mlp_sizes(sh, 1, D, sh["F"], "shared expert")
    return Mlp(sh["fmt"], sh["F"], _ptr(sh["wg"]), _ptr(sh["wu"]), _ptr(sh["wd"]),
               _ptr(sh["sg"]), _ptr(sh["su"]), _ptr(sh["sd"]), int(sh.get("layout", LAYOUT_ROWS)),
               int(sh.get("gs", 0)))


# ------------------------------------------------------------------ tiled layout
def tiled_bytes(fmt: int, count: int, O: int, I: int) -> int:
    return int(lib().coli_tiled_bytes(fmt, count, O, I))


def pack_tiled(fmt: int, W: torch.Tensor, count: int, O: int, I: int, dst: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """The tiled copy of `count` stacked row-major [O, I] matrices (uint8)."""
    nb = tiled_bytes(fmt, count, O, I)
    if nb < 0:
        raise ColiError(ESHAPE, "coli_tiled_bytes")
    if dst is None:
        dst = torch.empty((max(nb, 16),), dtype=torch.uint8, device=W.device)
    _need(W, count * O * row_bytes(fmt, I), "pack_tiled W")
    _need(dst, nb, "pack_tiled dst")
    rc = lib().coli_pack_tiled(fmt, _ptr(W), count, O, I, _ptr(dst), _stream(stream))
    _check(rc, "coli_pack_tiled")
    return dst


def pack_tiled_grouped(W: torch.Tensor, count: int, O: int, I: int, dst: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """The grouped tiled copy of `count` stacked row-major int4 [O, I]
    matrices (uint8)."""
    nb = tiled_bytes(I4, count, O, I)
    if nb < 0:
        raise ColiError(ESHAPE, "coli_tiled_bytes")
    if dst is None:
        dst = torch.empty((max(nb, 16),), dtype=torch.uint8, device=W.device)
    _need(W, count * O * row_bytes(I4, I), "pack_tiled_grouped W")
    _need(dst, nb, "pack_tiled_grouped dst")
    rc = lib().coli_pack_tiled_grouped(_ptr(W), count, O, I, _ptr(dst), _stream(stream))
    _check(rc, "coli_pack_tiled_grouped")
    return dst


def grouped_scale_bytes(count: int, O: int, I: int, gs: int) -> int:
    return int(lib().coli_grouped_scale_bytes(count, O, I, gs))


def pack_scales_grouped(S: torch.Tensor, count: int, O: int, I: int, gs: int,
                        dst: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Group scales [count, O, ceil(I / gs)] fp32 packed per 16-row tile and
    group (float32 tensor of grouped_scale_bytes / 4 elements)."""
    nb = grouped_scale_bytes(count, O, I, gs)
    if nb < 0:
        raise ColiError(ERANGE, "coli_grouped_scale_bytes")
    if dst is None:
        dst = torch.empty((max(nb // 4, 4),), dtype=torch.float32, device=S.device)
    _need(S, 4 * count * O * ((I + gs - 1) // gs), "pack_scales_grouped S")
    _need(dst, nb, "pack_scales_grouped dst")
    rc = lib().coli_pack_scales_grouped(_ptr(S), count, O, I, gs, _ptr(dst), _stream(stream))
    _check(rc, "coli_pack_scales_grouped")
    return dst


def tile_mlps(ex: dict, D: int | None = None) -> dict:
    """A copy of an experts dict (stacked E experts) or of a shared-expert
    dict (one matrix each; pass the width D) with its weights in the tiled
    layout; the scales are the original tensors -- or, for grouped-scale
    int4 (a "gs" entry), weights and scales in the grouped tiled layout."""
    n = ex.get("E", 1)
    D = ex["D"] if D is None else D
    F = ex["F"]
    out = dict(ex)
    gs = int(ex.get("gs", 0))
    if gs:
        if ex["fmt"] != I4:
            raise ColiError(EFMT, "tile_mlps: grouped scales need int4")
        out["wg"] = pack_tiled_grouped(ex["wg"], n, F, D)
        out["wu"] = pack_tiled_grouped(ex["wu"], n, F, D)
        out["wd"] = pack_tiled_grouped(ex["wd"], n, D, F)
        out["sg"] = pack_scales_grouped(ex["sg"], n, F, D, gs)
        out["su"] = pack_scales_grouped(ex["su"], n, F, D, gs)
        out["sd"] = pack_scales_grouped(ex["sd"], n, D, F, gs)
        out["layout"] = LAYOUT_TILED_GROUPED
        return out
    out["wg"] = pack_tiled(ex["fmt"], ex["wg"], n, F, D)
    out["wu"] = pack_tiled(ex["fmt"], ex["wu"], n, F, D)
    out["wd"] = pack_tiled(ex["fmt"], ex["wd"], n, D, F)
    out["layout"] = LAYOUT_TILED
    return out


def moe_workspace_bytes(S, K, E, D, F, F_shared=0, prec=PREC_FP32) -> int:
    return int(lib().coli_moe_workspace_bytes(S, K, E, D, F, F_shared, prec))


def moe_workspace_layout(S, K, E, D, F, F_shared=0, prec=PREC_FP32) -> dict:
    L = WsLayout()
    rc = lib().coli_moe_workspace_layout(S, K, E, D, F, F_shared, prec, C.byref(L))
    _check(rc, "coli_moe_workspace_layout")
    return {n: getattr(L, n) for n, _ in WsLayout._fields_}


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    t = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def _check_layer_io(ex: dict, x, S: int, K: int, out, tensors_sk: dict):
    """x and out hold S rows of the experts' width; each routing tensor S K."""
    D = ex["D"]
    if x.dim() != 2 or x.shape[1] != D:
        raise ColiError(ESHAPE, f"x must be [S, {D}] (the experts' width), got {tuple(x.shape)}")
    _need(out, 4 * S * D, "out")
    for name, t in tensors_sk.items():
        _need(t, 4 * S * K, name)


def moe_gemv(ex: dict, x, idx, w, out=None, prec=PREC_FP32, ws=None, stream=None):
    S, D = x.shape
    K = idx.shape[1]
    if out is None:
        out = torch.empty((S, D), dtype=torch.float32, device=x.device)
    _check_layer_io(ex, x, S, K, out, {"idx": idx, "w": w})
    es = experts_struct(ex)
    nb = moe_workspace_bytes(S, K, ex["E"], D, ex["F"], 0, prec)
    if ws is None:
        ws = alloc_workspace(nb, x.device)
    rc = lib().coli_moe_gemv(C.byref(es), _ptr(x), S, K, _ptr(idx), _ptr(w), _ptr(out), prec,
                             _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "coli_moe_gemv")
    return out, ws


def _router_struct(router_p, K):
    return RouterParams(_ptr(router_p["w"]) if router_p else None,
                        _ptr(router_p["bias"]) if router_p else None, K,
                        int(router_p.get("norm_topk", 1)) if router_p else 1,
                        float(router_p.get("routed_scale", 2.5)) if router_p else 1.0,
                        float(router_p.get("topp", 0.0)) if router_p else 0.0)


def moe_layer_tail(router_p: dict | None, ex: dict, shared: dict | None, x, norm_w, eps: float,
                   pre_idx=None, pre_w=None, out=None, idx_out=None, w_out=None, prec=PREC_FP32,
                   ws=None, K=None, stream=None):
    """out = x + moe_layer(rmsnorm(x)); out may be x (in place)."""
    S, D = x.shape
    if K is None:
        K = router_p["K"] if router_p else pre_idx.shape[1]
    if out is None:
        out = torch.empty((S, D), dtype=torch.float32, device=x.device)
    _check_layer_io(ex, x, S, K, out, {"pre_idx": pre_idx, "pre_w": pre_w, "idx_out": idx_out,
                                       "w_out": w_out})
    _need(norm_w, 4 * D, "norm_w")
    rp = _router_struct(router_p, K)
    es = experts_struct(ex)
    sp = C.byref(mlp_struct(shared, D)) if shared is not None else None
    Fs = shared["F"] if shared is not None else 0
    if ws is None:
        ws = alloc_workspace(moe_workspace_bytes(S, K, ex["E"], D, ex["F"], Fs, prec), x.device)
    rc = lib().coli_moe_layer_tail(C.byref(rp), C.byref(es), sp, _ptr(x), _ptr(norm_w), float(eps), S,
                                   _ptr(pre_idx), _ptr(pre_w), _ptr(out), _ptr(idx_out), _ptr(w_out),
                                   prec, _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "coli_moe_layer_tail")
    return out, ws


def moe_layer(router_p: dict | None, ex: dict, shared: dict | None, x, pre_idx=None, pre_w=None,
              out=None, idx_out=None, w_out=None, prec=PREC_FP32, ws=None, K=None, stream=None):
    S, D = x.shape
    if K is None:
        K = router_p["K"] if router_p else pre_idx.shape[1]
    if out is None:
        out = torch.empty((S, D), dtype=torch.float32, device=x.device)
    _check_layer_io(ex, x, S, K, out, {"pre_idx": pre_idx, "pre_w": pre_w, "idx_out": idx_out,
                                       "w_out": w_out})
    rp = _router_struct(router_p, K)
    es = experts_struct(ex)
    sp = C.byref(mlp_struct(shared, D)) if shared is not None else None
    Fs = shared["F"] if shared is not None else 0
    nb = moe_workspace_bytes(S, K, ex["E"], D, ex["F"], Fs, prec)
    if ws is None:
        ws = alloc_workspace(nb, x.device)
    rc = lib().coli_moe_layer(C.byref(rp), C.byref(es), sp, _ptr(x), S, _ptr(pre_idx),
                              _ptr(pre_w), _ptr(out), _ptr(idx_out), _ptr(w_out), prec,
                              _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "coli_moe_layer")
    return out, ws


def moe_layer_noalloc(router_p: dict | None, ex: dict, shared: dict | None, x, out, pre_idx=None,
                      pre_w=None, idx_out=None, w_out=None, prec=PREC_FP32, K=None, stream=None) -> int:
    """coli_moe_layer on the library's static scratch: the caller passes every
    input and output (out included); nothing is allocated.  Returns the
    status code."""
    S, D = x.shape
    if K is None:
        K = router_p["K"] if router_p else pre_idx.shape[1]
    _check_layer_io(ex, x, S, K, out, {"pre_idx": pre_idx, "pre_w": pre_w, "idx_out": idx_out,
                                       "w_out": w_out})
    rp = _router_struct(router_p, K)
    es = experts_struct(ex)
    sp = C.byref(mlp_struct(shared, D)) if shared is not None else None
    return int(lib().coli_moe_layer_noalloc(C.byref(rp), C.byref(es), sp, _ptr(x), S, _ptr(pre_idx),
                                            _ptr(pre_w), _ptr(out), _ptr(idx_out), _ptr(w_out), prec,
                                            _stream(stream)))


def stage_timing(enable: bool) -> None:
    _check(lib().coli_stage_timing(1 if enable else 0), "coli_stage_timing")


def stage_times(reset: bool = True) -> dict:
    """{stage name: (total ms, launches)} since the last reset (waits for the
    recorded events)."""
    ms = (C.c_double * NSTAGES)()
    calls = (C.c_int64 * NSTAGES)()
    _check(lib().coli_stage_times(ms, calls, 1 if reset else 0), "coli_stage_times")
    return {lib().coli_stage_name(i).decode(): (ms[i], calls[i]) for i in range(NSTAGES)}


def check_device_flags(ws, stream=None) -> tuple[int, int]:
    f = C.c_uint32(0)
    rc = lib().coli_check_device_flags(_ptr(ws), _stream(stream), C.byref(f))
    return rc, f.value
