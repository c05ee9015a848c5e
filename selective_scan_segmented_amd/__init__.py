"""selective_scan_segmented_amd -- SF-Mamba's folded, segmented selective scan on MI355X.

The compute lives in ``libsfm.so`` (hand-written HIP kernels for gfx950 behind
the C ABI declared in ``include/sfm.h``).  This module is the thin Python
binding: it checks tensors, passes their device pointers and the current HIP
stream, and turns non-zero status codes into exceptions.  Every step runs in
the library's kernels; there is no fallback -- if ``libsfm.so`` is missing the
first call raises.

Functions keep the C names:
  sfm_selective_scan_fwd, sfm_dwconv1d_fold, sfm_aux_pad_swap, sfm_pick_b1
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["sfm_selective_scan_fwd", "sfm_selective_scan_fwd_ex", "sfm_selective_scan_fwd_ws",
           "sfm_selective_scan_fwd_ws_size", "sfm_selective_scan_bwd",
           "sfm_selective_scan_bwd_workspace_size", "sfm_dwconv1d_fold", "sfm_aux_pad_swap", "sfm_aux_pad_bwd",
           "sfm_aux_pad_bwd_ex",
           "sfm_pick_b1", "sfm_scan_plan_string", "sfm_version", "library_path", "load_library", "SFMError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libsfm.so")
_lib = None

SFM_F32, SFM_BF16 = 0, 1
SFM_AUX_PAD, SFM_AUX_SWAP = 0, 1
_ACT = {None: 0, "none": 0, "silu": 1, 0: 0, 1: 1}


class SFMError(RuntimeError):
    pass


def library_path() -> str:
    return _LIBPATH


def load_library():
    """Load libsfm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        raise ImportError(f"libsfm.so not found at {_LIBPATH}; build it with "
                          "`python -m selective_scan_segmented_amd.build`")
    lib = ctypes.CDLL(_LIBPATH)
    vp, i64, ci, fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.sfm_selective_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, fp, ci, fp, fp, ci, ci, ci, vp,
                                           i64, i64, i64, i64, i64, ci, vp]
    lib.sfm_selective_scan_fwd_ex.argtypes = [vp, vp, fp, vp, vp, fp, fp, ci, fp, fp, ci, ci, ci, vp,
                                              i64, i64, i64, i64, i64, ci, ci, vp]
    lib.sfm_selective_scan_fwd_ws.argtypes = [vp, vp, fp, vp, vp, fp, fp, ci, fp, fp, ci, ci, ci, vp,
                                              i64, i64, i64, i64, i64, ci, ci, vp, i64, vp]
    lib.sfm_selective_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, fp, ci, fp, fp, ci, ci, ci, vp,
                                                   i64, i64, i64, i64, i64, ci, ci, vp]
    lib.sfm_selective_scan_fwd_ws_size.argtypes = [i64, i64, i64, i64, i64, ci, ci, ci,
                                                   ctypes.POINTER(ctypes.c_int64)]
    lib.sfm_dwconv1d_fold.argtypes = [vp, fp, fp, vp, i64, i64, i64, i64, ci, ci, ci, ci, vp]
    lib.sfm_selective_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, fp, ci, fp, fp, ci, ci, ci, vp,
                                           vp, vp, fp, fp, fp, fp, fp, fp, fp,
                                           i64, i64, i64, i64, i64, ci, ci, vp, i64, vp]
    lib.sfm_selective_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, ci, ci, ci,
                                                          ctypes.POINTER(ctypes.c_int64)]
    lib.sfm_aux_pad_bwd.argtypes = [vp, vp, i64, i64, i64, ci, vp]
    lib.sfm_aux_pad_bwd_ex.argtypes = [vp, vp, i64, i64, i64, ci, ci, vp]
    lib.sfm_aux_pad_swap.argtypes = [vp, vp, i64, i64, i64, ci, ci, vp]
    lib.sfm_pick_b1.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.sfm_scan_plan_string.argtypes = [i64, i64, i64, i64, i64, ci, ci, ci, ctypes.c_char_p, i64]
    for f in ("sfm_selective_scan_fwd", "sfm_selective_scan_fwd_ex", "sfm_selective_scan_fwd_ws",
              "sfm_selective_scan_fwd_ws_size", "sfm_dwconv1d_fold", "sfm_aux_pad_swap",
              "sfm_pick_b1", "sfm_version", "sfm_scan_plan_string", "sfm_selective_scan_bwd",
              "sfm_selective_scan_bwd_workspace_size", "sfm_aux_pad_bwd", "sfm_aux_pad_bwd_ex"):
        getattr(lib, f).restype = ctypes.c_int
    lib.sfm_status_string.argtypes = [ctypes.c_int]
    lib.sfm_status_string.restype = ctypes.c_char_p
    lib.sfm_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int, name: str):
    if rc != 0:
        lib = load_library()
        raise SFMError(f"{name}: {lib.sfm_status_string(rc).decode()} ({rc}): {lib.sfm_last_error().decode()}")


def sfm_version() -> int:
    return load_library().sfm_version()


def _torch():
    import torch
    return torch


def _io_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SFM_F32
    if t.dtype == torch.bfloat16:
        return SFM_BF16
    raise TypeError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


SFM_FUSE_PAD, SFM_FUSE_SWAP, SFM_LAYOUT_BLD = 1, 2, 4
SFM_NOALLOC_SCRATCH_BYTES = 32 << 20  # static scratch of sfm_selective_scan_fwd_noalloc (include/sfm.h)


def sfm_selective_scan_fwd(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, delta_softplus=True,
                           conv_w=None, conv_b=None, conv_pad_left=1, conv_act=None, y=None, B2=1,
                           stream=None):
    """Folded, segmented selective scan (see include/sfm.h).

    u, delta: [B, D, L]; A: [D, N] float32; Bm, Cm: [B, N, L]; io dtype float32 or bfloat16.
    With conv_w ([D, K] float32) ``u`` is the conv input and the boundary-masked conv is fused.
    B2 samples form one folded row (B1 = B / B2).  Returns y [B, D, L] (allocated if None).
    """
    return sfm_selective_scan_fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b,
                                     conv_pad_left, conv_act, y, B2, 0, stream)


def sfm_selective_scan_fwd_ex(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, delta_softplus=True,
                              conv_w=None, conv_b=None, conv_pad_left=1, conv_act=None, y=None, B2=1,
                              flags=0, stream=None):
    """sfm_selective_scan_fwd with the aux pad (flags & SFM_FUSE_PAD: u is the unpadded
    [B, D, L-2] stage input) and/or the aux swap of y (flags & SFM_FUSE_SWAP) fused in.
    flags & SFM_LAYOUT_BLD: channel-last tensors, u/delta/y [B, L, D] (u [B, L-2, D] with
    the pad), Bm/Cm [B, L, N]."""
    return _fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b, conv_pad_left,
                   conv_act, y, B2, flags, stream, False)


def _fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b, conv_pad_left, conv_act, y,
            B2, flags, stream, workspace):
    """Argument marshalling of the fused forward entry points (workspace False:
    sfm_selective_scan_fwd_ex; "noalloc": sfm_selective_scan_fwd_noalloc; else
    sfm_selective_scan_fwd_ws)."""
    torch = _torch()
    io = _io_code(u)
    cl = bool(flags & SFM_LAYOUT_BLD)
    if cl:
        B, XL, D = u.shape
    else:
        B, D, XL = u.shape
    L = XL + 2 if flags & SFM_FUSE_PAD else XL
    N = A.shape[1]
    if B % B2:
        raise ValueError(f"B2={B2} must divide B={B}")
    tl = (lambda a, b_: (B, b_, a)) if cl else (lambda a, b_: (B, a, b_))  # [B, a, b] in this layout
    _dev(u, "u")
    _dev(delta, "delta", u.dtype, tl(D, L))
    _dev(A, "A", torch.float32, (D, N))
    _dev(Bm, "Bm", u.dtype, tl(N, L))
    _dev(Cm, "Cm", u.dtype, tl(N, L))
    _dev(Dskip, "Dskip", torch.float32, (D,))
    _dev(delta_bias, "delta_bias", torch.float32, (D,))
    K = 0
    if conv_w is not None:
        _dev(conv_w, "conv_w", torch.float32)
        if conv_w.dim() != 2 or conv_w.shape[0] != D:
            raise ValueError("conv_w must be [D, K]")
        K = conv_w.shape[1]
        _dev(conv_b, "conv_b", torch.float32, (D,))
    if y is None:
        y = torch.empty(tl(D, L), dtype=u.dtype, device=u.device)
    _dev(y, "y", u.dtype, tl(D, L))
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(conv_w), _ptr(conv_b), K, int(conv_pad_left), _ACT[conv_act], _ptr(y),
            B // B2, B2, D, N, L, io, int(flags))
    if workspace is False:
        rc = load_library().sfm_selective_scan_fwd_ex(*args, _stream(stream))
    elif isinstance(workspace, str) and workspace == "noalloc":
        rc = load_library().sfm_selective_scan_fwd_noalloc(*args, _stream(stream))
    else:
        need = sfm_selective_scan_fwd_ws_size(B // B2, B2, D, N, L, K, "bf16" if io == SFM_BF16 else "f32",
                                              int(flags))
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=u.device)
        _dev(workspace, "workspace")
        rc = load_library().sfm_selective_scan_fwd_ws(*args, _ptr(workspace),
                                                      workspace.numel() * workspace.element_size(),
                                                      _stream(stream))
    _check(rc, "sfm_selective_scan_fwd")
    return y


def sfm_selective_scan_fwd_ws(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, delta_softplus=True,
                              conv_w=None, conv_b=None, conv_pad_left=1, conv_act=None, y=None, B2=1,
                              flags=0, workspace=None, stream=None):
    """sfm_selective_scan_fwd_ex with a device workspace (a uint8 GPU tensor of at least
    sfm_selective_scan_fwd_ws_size() bytes; allocated here when None): rows too long
    for the in-LDS carries are split along L across the whole GPU."""
    return _fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b, conv_pad_left,
                   conv_act, y, B2, flags, stream, workspace)


def sfm_selective_scan_fwd_noalloc(u, delta, A, Bm, Cm, Dskip=None, delta_bias=None, delta_softplus=True,
                                   conv_w=None, conv_b=None, conv_pad_left=1, conv_act=None, y=None, B2=1,
                                   flags=0, stream=None):
    """sfm_selective_scan_fwd_ws without a workspace argument: the library's static
    per-GPU scratch array stands in for it (see include/sfm.h for its limit).  ``y``
    must be passed by callers that cannot allocate (else it is allocated here)."""
    return _fwd_ex(u, delta, A, Bm, Cm, Dskip, delta_bias, delta_softplus, conv_w, conv_b, conv_pad_left,
                   conv_act, y, B2, flags, stream, "noalloc")


def sfm_selective_scan_fwd_ws_size(B1: int, B2: int, D: int, N: int, L: int, conv_k: int = 4,
                                   io: str = "bf16", flags: int = 0) -> int:
    """Workspace bytes sfm_selective_scan_fwd_ws needs (host only; 0: the regular forward runs)."""
    out = ctypes.c_int64(0)
    _check(load_library().sfm_selective_scan_fwd_ws_size(B1, B2, D, N, L, conv_k,
                                                         SFM_BF16 if io == "bf16" else SFM_F32, flags,
                                                         ctypes.byref(out)),
           "sfm_selective_scan_fwd_ws_size")
    return int(out.value)


def sfm_selective_scan_bwd_workspace_size(B1: int, B2: int, D: int, N: int, L: int, conv_k: int = 4,
                                          io: str = "bf16", flags: int = 0) -> int:
    """Workspace bytes sfm_selective_scan_bwd needs (host only)."""
    out = ctypes.c_int64(0)
    _check(load_library().sfm_selective_scan_bwd_workspace_size(B1, B2, D, N, L, conv_k,
                                                                SFM_BF16 if io == "bf16" else SFM_F32, flags,
                                                                ctypes.byref(out)),
           "sfm_selective_scan_bwd_workspace_size")
    return int(out.value)


def sfm_selective_scan_bwd(u, delta, A, Bm, Cm, dy, Dskip=None, delta_bias=None, delta_softplus=True,
                           conv_w=None, conv_b=None, conv_pad_left=1, conv_act=None, B2=1, flags=0,
                           workspace=None, grads=None, stream=None):
    """Gradients of sfm_selective_scan_fwd_ex for upstream dy (see include/sfm.h).

    Returns a dict: du (padded layout [B, D, L], io), ddelta (io), dA, dBm, dCm,
    dDskip, ddelta_bias, dconv_w, dconv_b (float32).  `grads` may hold
    preallocated tensors under those names; `workspace` a uint8 GPU tensor of at
    least sfm_selective_scan_bwd_workspace_size() bytes.  flags & SFM_LAYOUT_BLD:
    channel-last tensors ([B, L, D] and [B, L, N], gradients likewise)."""
    torch = _torch()
    io = _io_code(u)
    cl = bool(flags & SFM_LAYOUT_BLD)
    if cl:
        B, XL, D = u.shape
    else:
        B, D, XL = u.shape
    L = XL + 2 if flags & SFM_FUSE_PAD else XL
    N = A.shape[1]
    if B % B2:
        raise ValueError(f"B2={B2} must divide B={B}")
    tl = (lambda a, b_: (B, b_, a)) if cl else (lambda a, b_: (B, a, b_))  # [B, a, b] in this layout
    _dev(u, "u")
    for t, name, shape in ((delta, "delta", tl(D, L)), (Bm, "Bm", tl(N, L)), (Cm, "Cm", tl(N, L)),
                           (dy, "dy", tl(D, L))):
        _dev(t, name, u.dtype, shape)
    _dev(A, "A", torch.float32, (D, N))
    _dev(Dskip, "Dskip", torch.float32, (D,))
    _dev(delta_bias, "delta_bias", torch.float32, (D,))
    K = 0
    if conv_w is not None:
        _dev(conv_w, "conv_w", torch.float32)
        if conv_w.dim() != 2 or conv_w.shape[0] != D:
            raise ValueError("conv_w must be [D, K]")
        K = conv_w.shape[1]
        _dev(conv_b, "conv_b", torch.float32, (D,))
    g = dict(grads or {})
    f32 = dict(dtype=torch.float32, device=u.device)
    shapes = dict(du=(tl(D, L), u.dtype), ddelta=(tl(D, L), u.dtype), dA=((D, N), torch.float32),
                  dBm=(tl(N, L), torch.float32), dCm=(tl(N, L), torch.float32))
    if Dskip is not None:
        shapes["dDskip"] = ((D,), torch.float32)
    if delta_bias is not None:
        shapes["ddelta_bias"] = ((D,), torch.float32)
    if conv_w is not None:
        shapes["dconv_w"] = ((D, K), torch.float32)
        if conv_b is not None:
            shapes["dconv_b"] = ((D,), torch.float32)
    for k, (shape, dt) in shapes.items():
        if g.get(k) is None:
            g[k] = torch.empty(shape, dtype=dt, device=u.device)
        _dev(g[k], k, dt, shape)
    need = sfm_selective_scan_bwd_workspace_size(B // B2, B2, D, N, L, K, "bf16" if io == SFM_BF16 else "f32",
                                                 flags)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=u.device)
    _dev(workspace, "workspace")
    rc = load_library().sfm_selective_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(delta_bias), int(bool(delta_softplus)),
        _ptr(conv_w), _ptr(conv_b), K, int(conv_pad_left), _ACT[conv_act], _ptr(dy),
        _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dBm"]), _ptr(g["dCm"]), _ptr(g.get("dDskip")),
        _ptr(g.get("ddelta_bias")), _ptr(g.get("dconv_w")), _ptr(g.get("dconv_b")),
        B // B2, B2, D, N, L, io, int(flags), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(rc, "sfm_selective_scan_bwd")
    return g


def sfm_aux_pad_bwd(gpad, gx=None, stream=None):
    """Gradient of the aux pad: gpad [B, D, T+2] -> gx [B, D, T]."""
    return sfm_aux_pad_bwd_ex(gpad, gx, 0, stream)


def sfm_aux_pad_bwd_ex(gpad, gx=None, flags=0, stream=None):
    """Gradient of the aux pad; flags & SFM_LAYOUT_BLD: gpad [B, T+2, D] -> gx [B, T, D]."""
    io = _io_code(gpad)
    cl = bool(flags & SFM_LAYOUT_BLD)
    if cl:
        B, L, D = gpad.shape
        shape = (B, L - 2, D)
    else:
        B, D, L = gpad.shape
        shape = (B, D, L - 2)
    _dev(gpad, "gpad")
    if gx is None:
        gx = _torch().empty(shape, dtype=gpad.dtype, device=gpad.device)
    _dev(gx, "gx", gpad.dtype, shape)
    _check(load_library().sfm_aux_pad_bwd_ex(_ptr(gpad), _ptr(gx), B, D, L - 2, io, int(flags), _stream(stream)),
           "sfm_aux_pad_bwd")
    return gx


def sfm_dwconv1d_fold(x, w, bias=None, pad_left=1, act=None, out=None, B2=1, stream=None):
    """Boundary-masked depthwise conv1d over folded rows: x [B, D, L], w [D, K] float32."""
    torch = _torch()
    io = _io_code(x)
    B, D, L = x.shape
    if B % B2:
        raise ValueError(f"B2={B2} must divide B={B}")
    _dev(x, "x")
    _dev(w, "w", torch.float32)
    if w.dim() != 2 or w.shape[0] != D:
        raise ValueError("w must be [D, K]")
    _dev(bias, "bias", torch.float32, (D,))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (B, D, L))
    rc = load_library().sfm_dwconv1d_fold(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), B // B2, B2, D, L, w.shape[1],
                                          int(pad_left), _ACT[act], io, _stream(stream))
    _check(rc, "sfm_dwconv1d_fold")
    return out


def sfm_aux_pad_swap(inp, out=None, mode="pad", stream=None):
    """mode 'pad': [B, D, T] -> [B, D, T+2] with mean-initialised ends;
    mode 'swap': [B, D, L] -> ends exchanged (in place when ``out is inp``)."""
    torch = _torch()
    io = _io_code(inp)
    B, D, n = inp.shape
    _dev(inp, "in")
    if mode == "pad":
        T, code = n, SFM_AUX_PAD
        if out is None:
            out = torch.empty((B, D, T + 2), dtype=inp.dtype, device=inp.device)
        _dev(out, "out", inp.dtype, (B, D, T + 2))
    elif mode == "swap":
        T, code = n - 2, SFM_AUX_SWAP
        if out is None:
            out = torch.empty_like(inp)
        _dev(out, "out", inp.dtype, (B, D, n))
    else:
        raise ValueError(f"mode must be 'pad' or 'swap', got {mode!r}")
    rc = load_library().sfm_aux_pad_swap(_ptr(inp), _ptr(out), B, D, T, code, io, _stream(stream))
    _check(rc, "sfm_aux_pad_swap")
    return out


def sfm_scan_plan_string(B1: int, B2: int, D: int, N: int, L: int, conv_k: int = 4, io: str = "bf16",
                         flags: int = 0) -> str:
    """The launch plan sfm_selective_scan_fwd(_ex) would use for these sizes (host only)."""
    buf = ctypes.create_string_buffer(256)
    _check(load_library().sfm_scan_plan_string(B1, B2, D, N, L, conv_k, SFM_BF16 if io == "bf16" else SFM_F32,
                                               flags, buf, 256), "sfm_scan_plan_string")
    return buf.value.decode()


def sfm_pick_b1(B: int, L: int, D: int, N: int) -> int:
    """Adaptive B1 from the offline table (host only); B2 = B // result."""
    out = ctypes.c_int64(0)
    _check(load_library().sfm_pick_b1(B, L, D, N, ctypes.byref(out)), "sfm_pick_b1")
    return int(out.value)
