"""CPU oracle for the folded, segmented selective scan (fp64, scalar loops).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg are the only users.  The product path (the HIP
library and its Python binding) never imports this package, and this package
never imports the product path.

The arithmetic lives in ``sfm_oracle.c`` (plain C, built with
``-O2 -ffp-contract=off``); this module only marshals float64 numpy arrays.
Every function takes float64 arrays holding the exact values of the io tensors
(bf16 / f32 inputs upcast exactly) and returns float64 results.

Page citations for each function are in ``sfm_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfm_oracle.c")
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_IO = {"f64": 0, "f32": 1, "bf16": 2}
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build() -> str:
    """Compile liboracle.so next to its source (gcc, no fast-math, no FMA contraction)."""
    tmp = _LIBPATH + ".tmp"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                           "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIBPATH)
    return _LIBPATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            build()
        lib = ctypes.CDLL(_LIBPATH)
        lib.oracle_aux_pad.argtypes = [_dp, _dp, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_aux_swap.argtypes = [_dp, _dp, _i64, _i64, _i64]
        lib.oracle_dwconv1d.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                        ctypes.c_int, ctypes.c_int]
        lib.oracle_selective_scan.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, _dp,
                                              _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_selective_scan_folded.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                                     _dp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_round_io.argtypes = [_dp, _dp, _i64, ctypes.c_int]
        lib.oracle_selective_scan_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                                  _dp, _dp, _i64, _i64, ctypes.c_int, _dp,
                                                  _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                                  _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_aux_pad_bwd.argtypes = [_dp, _dp, _i64, _i64, _i64]
        lib.oracle_threads.argtypes = [ctypes.c_int]
        for f in ("oracle_aux_pad", "oracle_aux_swap", "oracle_dwconv1d", "oracle_selective_scan",
                  "oracle_selective_scan_folded", "oracle_round_io", "oracle_threads",
                  "oracle_selective_scan_bwd", "oracle_aux_pad_bwd"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (code {rc})")


def threads(n: int = 0) -> int:
    """Set the OpenMP thread count (n > 0) and return the count in effect."""
    return _load().oracle_threads(n)


def round_io(a, io: str) -> np.ndarray:
    """Round float64 values to the io type (round to nearest even), kept as float64."""
    a = _f64(a)
    out = np.empty_like(a)
    _check(_load().oracle_round_io(_ptr(a), _ptr(out), a.size, _IO[io]), "round_io")
    return out


def aux_pad(x, io: str = "f64") -> np.ndarray:
    """x [B, D, T] -> [B, D, T+2]; both ends = index-order float64 mean rounded once to io."""
    x = _f64(x)
    B, D, T = x.shape
    out = np.empty((B, D, T + 2))
    _check(_load().oracle_aux_pad(_ptr(x), _ptr(out), B, D, T, _IO[io]), "aux_pad")
    return out


def aux_swap(y) -> np.ndarray:
    """[B, D, L] -> same with positions 0 and L-1 exchanged."""
    y = _f64(y)
    B, D, L = y.shape
    out = np.empty_like(y)
    _check(_load().oracle_aux_swap(_ptr(y), _ptr(out), B, D, L), "aux_swap")
    return out


def dwconv1d(x, w, bias=None, pad_left: int = 1, act: int = 0, nthreads: int = 1) -> np.ndarray:
    """Per-sample zero-padded depthwise conv1d: x [B, D, L], w [D, K], bias [D] or None."""
    x, w = _f64(x), _f64(w)
    bias = None if bias is None else _f64(bias)
    B, D, L = x.shape
    K = w.shape[1]
    out = np.empty_like(x)
    _check(_load().oracle_dwconv1d(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), B, D, L, K, pad_left,
                                   act, nthreads), "dwconv1d")
    return out


def selective_scan(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, softplus: bool = True,
                   nthreads: int = 1) -> np.ndarray:
    """Per-sample selective scan; u, delta [B, D, L]; A [D, N]; Bm, Cm [B, N, L]."""
    u, delta, A, Bm, Cm = map(_f64, (u, delta, A, Bm, Cm))
    Dskip = None if Dskip is None else _f64(Dskip)
    delta_bias = None if delta_bias is None else _f64(delta_bias)
    B, D, L = u.shape
    N = A.shape[1]
    y = np.empty_like(u)
    _check(_load().oracle_selective_scan(_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                                         _ptr(delta_bias), int(softplus), _ptr(y), B, D, N, L, nthreads),
           "selective_scan")
    return y


def selective_scan_folded(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, softplus: bool = True,
                          B2: int = 1, nthreads: int = 1) -> np.ndarray:
    """Same result computed over folded rows [B1, D, B2*L] with the periodic reset."""
    u, delta, A, Bm, Cm = map(_f64, (u, delta, A, Bm, Cm))
    Dskip = None if Dskip is None else _f64(Dskip)
    delta_bias = None if delta_bias is None else _f64(delta_bias)
    B, D, L = u.shape
    if B % B2:
        raise ValueError("B2 must divide B")
    N = A.shape[1]
    y = np.empty_like(u)
    _check(_load().oracle_selective_scan_folded(_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                                _ptr(Dskip), _ptr(delta_bias), int(softplus), _ptr(y),
                                                B // B2, B2, D, N, L, nthreads), "selective_scan_folded")
    return y


def layer(x_padded, delta, A, Bm, Cm, Dskip, delta_bias, conv_w, conv_b=None, pad_left: int = 1,
          act: int = 0, softplus: bool = True, nthreads: int = 1, io: str = "f64"):
    """One scan layer on the padded sequence: u = conv(x); y = scan(u).

    ``io`` gives the precision the conv output is held in between the two steps
    when they run as separate launches; the fused launch keeps u in float32
    registers, which corresponds to io='f64' here up to float32 rounding."""
    u = dwconv1d(x_padded, conv_w, conv_b, pad_left=pad_left, act=act, nthreads=nthreads)
    if io != "f64":
        u = round_io(u, io)
    return selective_scan(u, delta, A, Bm, Cm, Dskip, delta_bias, softplus=softplus, nthreads=nthreads)


def selective_scan_bwd(x, delta, A, Bm, Cm, Dskip, delta_bias, dy, conv_w=None, conv_b=None,
                       pad_left: int = 1, act: int = 0, softplus: bool = True, nthreads: int = 1) -> dict:
    """Gradients of the per-sample layer (optional conv, then scan) for upstream dy.

    x is the conv input (or u without conv), [B, D, L].  Returns float64 arrays:
    dx [B,D,L], ddelta [B,D,L], dA [D,N], dBm, dCm [B,N,L], dDskip [D],
    ddelta_bias [D], and with conv dconv_w [D,K], dconv_b [D]."""
    x, delta, A, Bm, Cm, dy = map(_f64, (x, delta, A, Bm, Cm, dy))
    Dskip = None if Dskip is None else _f64(Dskip)
    delta_bias = None if delta_bias is None else _f64(delta_bias)
    B, D, L = x.shape
    N = A.shape[1]
    K = 0
    if conv_w is not None:
        conv_w = _f64(conv_w)
        K = conv_w.shape[1]
        conv_b = None if conv_b is None else _f64(conv_b)
    out = dict(dx=np.empty_like(x), ddelta=np.empty_like(x), dA=np.empty_like(A), dBm=np.empty_like(Bm),
               dCm=np.empty_like(Cm), dDskip=np.empty(D), ddelta_bias=np.empty(D))
    if conv_w is not None:
        out["dconv_w"] = np.empty_like(conv_w)
        out["dconv_b"] = np.empty(D)
    _check(_load().oracle_selective_scan_bwd(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(delta_bias), int(softplus),
        _ptr(conv_w), _ptr(conv_b), K, pad_left, act, _ptr(dy),
        _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dBm"]), _ptr(out["dCm"]),
        _ptr(out["dDskip"]), _ptr(out["ddelta_bias"]), _ptr(out.get("dconv_w")), _ptr(out.get("dconv_b")),
        B, D, N, L, nthreads), "selective_scan_bwd")
    return out


def aux_pad_bwd(dxp) -> np.ndarray:
    """Gradient of the aux pad: [B, D, T+2] -> [B, D, T]."""
    dxp = _f64(dxp)
    B, D, L = dxp.shape
    dx = np.empty((B, D, L - 2))
    _check(_load().oracle_aux_pad_bwd(_ptr(dxp), _ptr(dx), B, D, L - 2), "aux_pad_bwd")
    return dx


def layer_bwd(x, delta, A, Bm, Cm, Dskip, delta_bias, dy, conv_w=None, conv_b=None, pad_left: int = 1,
              act: int = 0, softplus: bool = True, fuse_pad: bool = False, fuse_swap: bool = False,
              nthreads: int = 1) -> dict:
    """Backward of pad (optional) -> conv -> scan -> swap (optional).

    With fuse_pad, x is the unpadded [B, D, L-2] stage input (its padded form
    is rebuilt exactly as the forward does, mean unrounded) and dx comes back
    unpadded; with fuse_swap, dy is the gradient of the swapped output."""
    x, dy = _f64(x), _f64(dy)
    xp = aux_pad(x, "f64") if fuse_pad else x
    if fuse_swap:
        dy = aux_swap(dy)
    g = selective_scan_bwd(xp, delta, A, Bm, Cm, Dskip, delta_bias, dy, conv_w, conv_b, pad_left, act,
                           softplus, nthreads)
    if fuse_pad:
        g["dx"] = aux_pad_bwd(g["dx"])
    return g
