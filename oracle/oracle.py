"""ctypes front end of the CPU oracle (coli_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It takes host numpy
arrays and returns fp64 numpy arrays; the arithmetic lives in coli_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.c")
_LIB = os.path.join(_HERE, "libcoli_oracle.so")

F32, I8, I4, I2 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile coli_oracle.c with gcc (IEEE fp64, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        vp, i32, i64, dp = C.c_void_p, C.c_int, C.c_int64, C.c_double
        L.cor_row_bytes.restype = i64
        L.cor_row_bytes.argtypes = [i32, i64]
        L.cor_unpack.restype = dp
        L.cor_unpack.argtypes = [i32, vp, i64]
        L.cor_num_threads.restype = i32
        L.cor_set_threads.restype = i32
        L.cor_set_threads.argtypes = [i32]
        L.cor_qgemv.restype = i32
        L.cor_qgemv.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.cor_qgemv_d.restype = i32
        L.cor_qgemv_d.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.cor_router.restype = i32
        L.cor_router.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, dp, dp,
                                 vp, vp, vp, vp, vp]
        L.cor_moe.restype = i32
        L.cor_moe.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, i64,
                              vp, vp, vp, vp, vp, vp]
        L.cor_qgemv_grouped.restype = i32
        L.cor_qgemv_grouped.argtypes = [vp, vp, i32, vp, i32, i32, i32, vp, vp]
        L.cor_qrow_i8.restype = C.c_float
        L.cor_qrow_i8.argtypes = [vp, i32, vp]
        L.cor_moe_idot.restype = i32
        L.cor_moe_idot.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i64, vp, vp, vp, vp]
        L.cor_qgemv_idot.restype = i32
        L.cor_qgemv_idot.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.cor_rmsnorm.restype = None
        L.cor_rmsnorm.argtypes = [vp, vp, i32, i32, C.c_float, vp]
        for name in ("cor_quantize_rows", "cor_pack_int4", "cor_pack_int2"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [vp, vp, vp, i32, i32, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().cor_num_threads())


def set_threads(n: int) -> int:
    """Host threads for later oracle calls; returns the previous count."""
    return int(lib().cor_set_threads(int(n)))


def row_bytes(fmt: int, I: int) -> int:
    return int(lib().cor_row_bytes(fmt, I))


def unpack(fmt: int, row: np.ndarray, i: int) -> float:
    row = np.ascontiguousarray(row)
    return float(lib().cor_unpack(fmt, _p(row), i))


def qgemv(fmt: int, W: np.ndarray, scale, x: np.ndarray, O: int | None = None):
    """y[s,o] = scale[o] * sum_i v(o,i) x[s,i] in fp64; returns (y, mag)."""
    x = np.atleast_2d(x)
    S, I = x.shape
    W = np.ascontiguousarray(W)
    if O is None:
        O = W.shape[0]
    assert W.nbytes >= O * row_bytes(fmt, I)
    sc = None if scale is None else _c(scale, np.float32)
    y = np.empty((S, O), np.float64)
    mag = np.empty((S, O), np.float64)
    if x.dtype == np.float64:
        xd = _c(x, np.float64)
        rc = lib().cor_qgemv_d(fmt, _p(W), _p(sc), _p(xd), S, I, O, _p(y), _p(mag))
    else:
        xf = _c(x, np.float32)
        rc = lib().cor_qgemv(fmt, _p(W), _p(sc), _p(xf), S, I, O, _p(y), _p(mag))
    assert rc == 0, rc
    return y, mag


def router(Wr, bias, x, K: int, norm_topk: int = 1, routed_scale: float = 2.5,
           topp: float = 0.0):
    """Returns dict(idx int32 [S,K], w fp64 [S,K], keff int32 [S],
    sig fp32 [S,E], logit fp64 [S,E])."""
    Wr = _c(Wr, np.float32)
    bias = _c(bias, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    E, D = Wr.shape
    S = x.shape[0]
    idx = np.empty((S, K), np.int32)
    w = np.empty((S, K), np.float64)
    keff = np.empty((S,), np.int32)
    sig = np.empty((S, E), np.float32)
    logit = np.empty((S, E), np.float64)
    rc = lib().cor_router(_p(Wr), _p(bias), _p(x), S, E, D, K, int(norm_topk),
                          float(routed_scale), float(topp), _p(idx), _p(w),
                          _p(keff), _p(sig), _p(logit))
    assert rc == 0, rc
    return dict(idx=idx, w=w, keff=keff, sig=sig, logit=logit)


class _Experts(C.Structure):
    _fields_ = [("fmt", C.c_int), ("E", C.c_int), ("D", C.c_int), ("F", C.c_int),
                ("wg", C.c_void_p), ("wu", C.c_void_p), ("wd", C.c_void_p),
                ("sg", C.c_void_p), ("su", C.c_void_p), ("sd", C.c_void_p), ("gs", C.c_int)]


class _Mlp(C.Structure):
    _fields_ = [("fmt", C.c_int), ("F", C.c_int),
                ("wg", C.c_void_p), ("wu", C.c_void_p), ("wd", C.c_void_p),
                ("sg", C.c_void_p), ("su", C.c_void_p), ("sd", C.c_void_p), ("gs", C.c_int)]


def moe(ex: dict, shared: dict | None, x, idx, w, intermediates: bool = False):
    """MoE output for S tokens.

    ex: dict(fmt, E, D, F, wg, wu, wd, sg, su, sd[, gs]) with host arrays
        stacked per expert ([E,F,rb(D)], [E,F,rb(D)], [E,D,rb(F)], [E,F],
        [E,F], [E,D]); with gs > 0 (int4 only) one scale per gs elements:
        sg, su [E,F,ceil(D/gs)], sd [E,D,ceil(F/gs)].
    shared: dict(fmt, F, wg, wu, wd, sg, su, sd[, gs]) or None.
    idx [S,K] int32 (entries < 0 skipped), w [S,K] (widened to fp64).
    Returns dict(out, mag) plus, when intermediates, per-pair rows
    (pair p = s*K + k; shared rows follow at S*K + s): h, g, u, gmag, umag, y.
    """
    x = _c(np.atleast_2d(x), np.float32)
    idx = _c(idx, np.int32)
    wd = _c(w, np.float64)
    S, K = idx.shape
    D, F = ex["D"], ex["F"]
    keep = [x, idx, wd]

    def arr(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return _p(a)

    e = _Experts(ex["fmt"], ex["E"], D, F, arr(ex["wg"]), arr(ex["wu"]), arr(ex["wd"]),
                 arr(_c(ex["sg"], np.float32)), arr(_c(ex["su"], np.float32)),
                 arr(_c(ex["sd"], np.float32)), int(ex.get("gs", 0)))
    sp = None
    if shared is not None:
        s = _Mlp(shared["fmt"], shared["F"], arr(shared["wg"]), arr(shared["wu"]),
                 arr(shared["wd"]), arr(_c(shared["sg"], np.float32)),
                 arr(_c(shared["su"], np.float32)), arr(_c(shared["sd"], np.float32)),
                 int(shared.get("gs", 0)))
        sp = C.pointer(s)
    out = np.empty((S, D), np.float64)
    mag = np.empty((S, D), np.float64)
    res = dict(out=out, mag=mag)
    rows = S * K + (S if shared is not None else 0)
    ptrs = [None] * 6
    if intermediates:
        Fi = F
        res.update(h=np.zeros((rows, Fi)), g=np.zeros((rows, Fi)), u=np.zeros((rows, Fi)),
                   gmag=np.zeros((rows, Fi)), umag=np.zeros((rows, Fi)),
                   y=np.zeros((rows, D)))
        ptrs = [_p(res[k]) for k in ("h", "g", "u", "gmag", "umag", "y")]
    rc = lib().cor_moe(C.byref(e), sp, _p(x), S, K, _p(idx), _p(wd), _p(out), _p(mag),
                       rows, *ptrs)
    assert rc == 0, rc
    return res


def moe_idot(ex: dict, shared: dict | None, x, idx, w, h_in=None):
    """MoE output on the pages' integer-dot path (int8 / int4 experts): x
    quantised per token, every product an exact integer dot with the pages'
    fp32 epilogue, h = silu(g) * u in fp32, quantised per row for the down
    product.  Arrays as for moe().  h_in: optional [S*K (+ S), F] fp32 rows
    (pair numbering) the down products quantise instead of the oracle's own h.
    Returns dict(out fp64 [S, D], h, g fp32 [rows, F], y fp32 [rows, D]);
    g is the gate product (the argument of silu)."""
    x = _c(np.atleast_2d(x), np.float32)
    idx = _c(idx, np.int32)
    wd = _c(w, np.float64)
    S, K = idx.shape
    D, F = ex["D"], ex["F"]
    keep = [x, idx, wd]

    def arr(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return _p(a)

    e = _Experts(ex["fmt"], ex["E"], D, F, arr(ex["wg"]), arr(ex["wu"]), arr(ex["wd"]),
                 arr(_c(ex["sg"], np.float32)), arr(_c(ex["su"], np.float32)),
                 arr(_c(ex["sd"], np.float32)), int(ex.get("gs", 0)))
    sp = None
    if shared is not None:
        sm = _Mlp(shared["fmt"], shared["F"], arr(shared["wg"]), arr(shared["wu"]),
                  arr(shared["wd"]), arr(_c(shared["sg"], np.float32)),
                  arr(_c(shared["su"], np.float32)), arr(_c(shared["sd"], np.float32)),
                 int(shared.get("gs", 0)))
        sp = C.pointer(sm)
    rows = S * K + (S if shared is not None else 0)
    hin = None
    if h_in is not None:
        hin = _c(h_in, np.float32)
        assert hin.shape == (rows, F)
    out = np.empty((S, D), np.float64)
    h = np.zeros((rows, F), np.float32)
    y = np.zeros((rows, D), np.float32)
    gv = np.zeros((rows, F), np.float32)
    rc = lib().cor_moe_idot(C.byref(e), sp, _p(x), S, K, _p(idx), _p(wd),
                            _p(hin) if hin is not None else None, rows, _p(out), _p(h), _p(y), _p(gv))
    assert rc == 0, rc
    return dict(out=out, h=h, y=y, g=gv)


def qgemv_grouped(W, scale, gs: int, x, O: int | None = None):
    """Grouped-scale int4 product (scale [O, ceil(I/gs)]); returns (y, mag) fp64."""
    W = _c(W, np.uint8)
    x = _c(np.atleast_2d(x), np.float32)
    S, I = x.shape
    O = W.shape[0] if O is None else O
    sc = _c(scale, np.float32)
    assert sc.size >= O * ((I + gs - 1) // gs)
    y = np.empty((S, O), np.float64)
    mag = np.empty((S, O), np.float64)
    rc = lib().cor_qgemv_grouped(_p(W), _p(sc), int(gs), _p(x), S, I, O, _p(y), _p(mag))
    assert rc == 0, rc
    return y, mag


def qrow_i8(x):
    """Per-row int8 quantisation of x [S, I] by absmax/127 (the pages' IDOT
    activations).  Returns (q int8 [S, I], s fp32 [S])."""
    x = _c(np.atleast_2d(x), np.float32)
    S, I = x.shape
    q = np.empty((S, I), np.int8)
    s = np.empty((S,), np.float32)
    for r in range(S):
        s[r] = lib().cor_qrow_i8(_p(x[r]), I, _p(q[r]))
    return q, s


def qgemv_idot(fmt: int, W, scale, x, O: int | None = None):
    """Integer-dot qgemv (int8 / int4 weights): returns (y fp32 [S, O], the
    exact integer dots int64 [S, O])."""
    W = _c(W, np.uint8)
    x = _c(np.atleast_2d(x), np.float32)
    S, I = x.shape
    O = W.shape[0] if O is None else O
    sc = _c(scale, np.float32)
    y = np.empty((S, O), np.float32)
    dot = np.empty((S, O), np.int64)
    rc = lib().cor_qgemv_idot(fmt, _p(W), _p(sc), _p(x), S, I, O, _p(y), _p(dot))
    assert rc == 0, rc
    return y, dot


def rmsnorm(x, w, eps: float):
    """Post-attention RMSNorm of each row of x [S, D] with weight w [D]
    (fp64 mean square, fp32 scale and products, as the pages define it).
    Returns fp32 [S, D]."""
    x = _c(np.atleast_2d(x), np.float32)
    w = _c(w, np.float32)
    S, D = x.shape
    assert w.shape == (D,)
    out = np.empty((S, D), np.float32)
    lib().cor_rmsnorm(_p(x), _p(w), S, D, float(eps), _p(out))
    return out


def layer_tail(x, norm_w, eps: float, ex: dict, shared: dict | None, idx, w):
    """The layer tail: out = x + moe(rmsnorm(x)) for given routing.
    Returns dict(out fp64 [S, D], mag fp64 [S, D] -- the MoE block's
    magnitude, the bound's scale -- and n fp32 [S, D], the normalised rows)."""
    n = rmsnorm(x, norm_w, eps)
    r = moe(ex, shared, n, idx, w)
    out = np.asarray(np.atleast_2d(x), np.float64) + r["out"]
    return dict(out=out, mag=r["mag"], n=n)


def quantize_rows(w, bits: int = 8):
    w = _c(np.atleast_2d(w), np.float32)
    O, I = w.shape
    q = np.empty((O, I), np.int8)
    s = np.empty((O,), np.float32)
    lib().cor_quantize_rows(_p(w), _p(q), _p(s), O, I, bits)
    return q, s


def pack_int4(w, bits: int = 4):
    w = _c(np.atleast_2d(w), np.float32)
    O, I = w.shape
    q = np.empty((O, (I + 1) // 2), np.uint8)
    s = np.empty((O,), np.float32)
    lib().cor_pack_int4(_p(w), _p(q), _p(s), O, I, bits)
    return q, s


def pack_int2(w, bits: int = 2):
    w = _c(np.atleast_2d(w), np.float32)
    O, I = w.shape
    q = np.empty((O, (I + 3) // 4), np.uint8)
    s = np.empty((O,), np.float32)
    lib().cor_pack_int2(_p(w), _p(q), _p(s), O, I, bits)
    return q, s
