"""Parity of the HIP backward (through the C ABI) against the float64 oracle backward.

Tolerance (|g - r| <= rtol (|r| + rms r), the forward's rule): the backward
runs the reverse recurrence and the per-position sums in float32 and adds the
per-tile / per-sample partial sums in a fixed order (a reduce launch), so its
float32 bar is 1e-4 (ten times the forward's 1e-5).  Outputs stored in bfloat16
(du, ddelta) keep the forward's 2e-2; float32 sums computed from bfloat16
inputs use 1e-3.
"""
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import from_dev, host_threads, to_dev

pytestmark = pytest.mark.gpu
NT = host_threads()
TOL = {"f32": {"io": 1e-4, "f32": 1e-4}, "bf16": {"io": 2e-2, "f32": 1e-3}}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def close(g, r, rtol, what):
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = rtol * (np.abs(r) + rms)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:4]
        raise AssertionError(f"{what}: {int(bad.sum())}/{r.size} outside rtol {rtol}; worst err/bound "
                             f"{float(np.max(err / np.maximum(bound, 1e-300))):.3g}; at {idx.tolist()}: got "
                             f"{[float(g[tuple(i)]) for i in idx]} want {[float(r[tuple(i)]) for i in idx]}")


def run_case(B, D, N, T, B2, K, P, act, softplus, flags, io, seed, use_conv=True, with_bias=True, cl=False):
    import torch
    w = synth.Workload("bwd", B=B, D=D, N=N, T=T, io=io, B2_list=(B2,), K=max(K, 1))
    li = synth.make_layer(w, seed=seed)
    L = T + 2
    rng = np.random.default_rng(seed + 99)
    dy32 = rng.standard_normal((B, D, L)).astype(np.float32)
    dy = synth.f32_to_bf16_bits(dy32) if io == "bf16" else dy32
    pad = bool(flags & sfm.SFM_FUSE_PAD)
    x_in = li.x if pad else None
    if not pad:
        # the conv input is a full [B, D, L] tensor when the pad is not fused
        xr = rng.standard_normal((B, D, L)).astype(np.float32)
        x_in = synth.f32_to_bf16_bits(xr) if io == "bf16" else xr
    f64 = (lambda a: synth.bf16_bits_to_f64(a)) if io == "bf16" else (lambda a: a.astype(np.float64))
    delta = li.delta
    if not softplus:
        # without softplus the step is delta + bias itself: keep it positive and small so the
        # recurrence decays (a negative step makes exp(Delta*A) grow without bound)
        with_bias = False
        d32 = (0.05 * np.abs(f64(li.delta))).astype(np.float32)
        delta = synth.f32_to_bf16_bits(d32) if io == "bf16" else d32
    conv_w = li.conv_w[:, :K] if use_conv else None
    dev = lambda a: to_dev(a)
    prm = dict(A=torch.from_numpy(li.A).cuda(),
               Dskip=torch.from_numpy(li.Dskip).cuda(),
               delta_bias=None)
    if with_bias:
        prm["delta_bias"] = torch.from_numpy(li.delta_bias).cuda()
    cw = torch.from_numpy(np.ascontiguousarray(conv_w)).cuda() if use_conv else None
    say(f"bwd case B={B} D={D} N={N} T={T} B2={B2} K={K} P={P} act={act} sp={softplus} flags={flags} io={io}")
    g = sfm.sfm_selective_scan_bwd(dev(x_in), dev(delta), prm["A"], dev(li.Bm), dev(li.Cm), dev(dy),
                                   Dskip=prm["Dskip"], delta_bias=prm["delta_bias"], delta_softplus=softplus,
                                   conv_w=cw, conv_pad_left=P, conv_act="silu" if act else None, B2=B2, flags=flags)
    torch.cuda.synchronize()
    if cl:
        # channel-last on the transposed tensors: the same kernel arithmetic and summation order
        tr = lambda a: a.transpose(1, 2).contiguous()
        gl = sfm.sfm_selective_scan_bwd(tr(dev(x_in)), tr(dev(delta)), prm["A"], tr(dev(li.Bm)), tr(dev(li.Cm)),
                                        tr(dev(dy)), Dskip=prm["Dskip"], delta_bias=prm["delta_bias"],
                                        delta_softplus=softplus, conv_w=cw, conv_pad_left=P,
                                        conv_act="silu" if act else None, B2=B2, flags=flags | sfm.SFM_LAYOUT_BLD)
        torch.cuda.synchronize()
        for k in g:
            a_ = from_dev(tr(gl[k])) if gl[k].dim() == 3 else from_dev(gl[k])
            assert np.array_equal(a_, from_dev(g[k])), f"channel-last {k} differs from channel-first"
    # oracle on the same bytes (padded input rebuilt with the io-rounded mean, as the forward uses)
    xo = f64(x_in)
    if pad:
        xo = oracle.aux_pad(xo, io)
    dyo = f64(dy)
    if flags & sfm.SFM_FUSE_SWAP:
        dyo = oracle.aux_swap(dyo)
    want = oracle.selective_scan_bwd(xo, f64(delta), li.A.astype(np.float64), f64(li.Bm), f64(li.Cm),
                                     li.Dskip.astype(np.float64),
                                     li.delta_bias.astype(np.float64) if with_bias else None, dyo,
                                     conv_w.astype(np.float64) if use_conv else None, None, P, act, softplus,
                                     nthreads=NT)
    t = TOL[io]
    close(from_dev(g["du"]), want["dx"], t["io"], "du")
    close(from_dev(g["ddelta"]), want["ddelta"], t["io"], "ddelta")
    for k in ("dA", "dBm", "dCm", "dDskip"):
        close(from_dev(g[k]), want[k], t["f32"], k)
    if with_bias:
        close(from_dev(g["ddelta_bias"]), want["ddelta_bias"], t["f32"], "ddelta_bias")
    if use_conv:
        close(from_dev(g["dconv_w"]), want["dconv_w"], t["f32"], "dconv_w")
    return g, want


@pytest.mark.parametrize("B2", [1, 2])
def test_bwd_tiny_f32(B2):
    run_case(B=4, D=16, N=4, T=8, B2=B2, K=4, P=1, act=0, softplus=True, flags=0, io="f32", seed=1)


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,sp,flags", [
    (3, 16, 4, 8, 1, 4, 1, 1, True, 0),       # SiLU conv
    (3, 16, 4, 8, 3, 4, 2, 0, False, 0),      # no softplus, folded row of three samples
    (2, 70, 5, 35, 1, 4, 0, 0, True, 0),      # partial channel tile, ragged last chunk, N padded to 8
    (2, 24, 16, 21, 2, 3, 1, 1, True, 0),     # N = 16 (4-position chunks)
    (2, 16, 8, 13, 1, 8, 3, 0, True, 0),      # widest conv
    (4, 16, 4, 8, 2, 4, 1, 0, True, 3),       # fused pad and swap
])
def test_bwd_variants_f32(B, D, N, T, B2, K, P, act, sp, flags):
    run_case(B=B, D=D, N=N, T=T, B2=B2, K=K, P=P, act=act, softplus=sp, flags=flags, io="f32", seed=B * 7 + T)


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,sp,flags", [
    (3, 72, 8, 14, 3, 4, 1, 1, True, 3),      # whole-sample kernel: partial tile of 8 rows, pad and swap
    (2, 16, 4, 8, 2, 4, 1, 0, True, 3),       # the same shape through both kernels
    (2, 24, 16, 21, 1, 4, 3, 0, True, 0),     # causal conv (lag 0), N = 16
])
@pytest.mark.parametrize("chunked", [False, True])
def test_bwd_kernels_f32(B, D, N, T, B2, K, P, act, sp, flags, chunked, monkeypatch):
    """Both backward kernels (whole-sample staging and chunk by chunk) on the same cases."""
    if chunked:
        monkeypatch.setenv("SFM_BWD_CHUNKED", "1")
    run_case(B=B, D=D, N=N, T=T, B2=B2, K=K, P=P, act=act, softplus=sp, flags=flags, io="f32", seed=B * 5 + T)


def test_bwd_stage4_bf16_chunked(monkeypatch):
    """The chunked kernel at the stage-4 shape (the default plan stages whole samples there)."""
    monkeypatch.setenv("SFM_BWD_CHUNKED", "1")
    run_case(B=64, D=640, N=8, T=49, B2=2, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=12)


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,sp,flags,segs,conv", [
    (2, 70, 5, 60, 1, 4, 1, 1, True, 3, 3, True),    # pad and swap, partial tile, N padded to 8
    (2, 24, 16, 45, 2, 4, 3, 0, True, 0, 4, True),   # causal conv (lag 0), N = 16, folded pairs
    (1, 16, 4, 40, 1, 8, 2, 0, True, 3, 5, True),    # widest window: 7 boundary positions, lag 5
    (2, 16, 8, 30, 1, 4, 0, 0, False, 0, 3, True),   # anti-causal side only (lag 3), no softplus
    (2, 16, 4, 30, 1, 1, 0, 0, True, 0, 4, False),   # no conv: no boundary partials
])
def test_bwd_split_rows_f32(B, D, N, T, B2, K, P, act, sp, flags, segs, conv, monkeypatch):
    """The chunked kernel with rows split along L (carry pass, composed carries,
    boundary partials) against the oracle; the plan must really split."""
    monkeypatch.setenv("SFM_BWD_CHUNKED", "1")
    kk = K if conv else 0
    whole = sfm.sfm_selective_scan_bwd_workspace_size(B // B2, B2, D, N, T + 2, kk, "f32", flags)
    monkeypatch.setenv("SFM_BWD_SEGMENTS", str(segs))
    split = sfm.sfm_selective_scan_bwd_workspace_size(B // B2, B2, D, N, T + 2, kk, "f32", flags)
    assert split > whole
    run_case(B=B, D=D, N=N, T=T, B2=B2, K=K, P=P, act=act, softplus=sp, flags=flags, io="f32", seed=B * 11 + T,
             use_conv=conv)


def test_bwd_split_rows_stage3_bf16():
    """The default plan splits rows when samples x tiles give few waves: stage-3
    rows (L = 198) for 4 samples and 320 channels, bfloat16, pad and swap."""
    run_case(B=4, D=320, N=8, T=196, B2=1, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=41)


def test_bwd_no_conv_f32():
    run_case(B=3, D=16, N=4, T=10, B2=1, K=1, P=0, act=0, softplus=True, flags=0, io="f32", seed=5,
             use_conv=False)


def test_bwd_no_bias_f32():
    run_case(B=2, D=16, N=4, T=6, B2=1, K=4, P=1, act=0, softplus=True, flags=0, io="f32", seed=6, with_bias=False)


def test_bwd_stage4_bf16_fused():
    """The bench's stage-4 layer shape, bf16, pad and swap fused."""
    run_case(B=256, D=640, N=8, T=49, B2=1, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=2)


def test_bwd_stage3_bf16():
    run_case(B=32, D=320, N=8, T=196, B2=2, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=3)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_pad_bwd(io):
    import torch
    rng = np.random.default_rng(4)
    B, D, T = 3, 70, 13
    g32 = rng.standard_normal((B, D, T + 2)).astype(np.float32)
    g = synth.f32_to_bf16_bits(g32) if io == "bf16" else g32
    f64 = synth.bf16_bits_to_f64(g) if io == "bf16" else g32.astype(np.float64)
    got = sfm.sfm_aux_pad_bwd(to_dev(g))
    torch.cuda.synchronize()
    close(from_dev(got), oracle.aux_pad_bwd(f64), 1e-6 if io == "f32" else 8e-3, "pad_bwd")


def test_bwd_workspace_too_small():
    import torch
    B, D, N, L = 2, 16, 4, 10
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda")
    with pytest.raises(sfm.SFMError):
        sfm.sfm_selective_scan_bwd(z(B, D, L), z(B, D, L), z(D, N), z(B, N, L), z(B, N, L), z(B, D, L),
                                   conv_w=z(D, 4), workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("chunked", [False, True])
def test_bwd_repeatable(chunked, monkeypatch):
    """The float32 sums are added in a fixed order: two calls give the same bits."""
    if chunked:
        monkeypatch.setenv("SFM_BWD_CHUNKED", "1")
    g1, _ = run_case(B=8, D=192, N=8, T=14, B2=2, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=21)
    g2, _ = run_case(B=8, D=192, N=8, T=14, B2=2, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=21)
    for k in ("du", "ddelta", "dA", "dBm", "dCm", "dDskip", "ddelta_bias", "dconv_w"):
        assert np.array_equal(from_dev(g1[k]), from_dev(g2[k])), k


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,sp,flags,io", [
    (2, 16, 4, 8, 2, 4, 1, 0, True, 3, "f32"),       # tiny, pad and swap, folded
    (3, 72, 5, 14, 3, 4, 1, 1, True, 3, "f32"),      # partial tile of 8 channels, SiLU conv, N padded
    (2, 24, 16, 21, 1, 4, 3, 0, True, 0, "f32"),     # causal conv, N = 16
    (3, 16, 8, 9, 1, 0, 0, 0, True, 2, "f32"),       # no conv, swap only
    (64, 640, 8, 49, 1, 4, 1, 0, True, 3, "bf16"),   # stage-4 shape (64 of its 256 samples)
    (2, 64, 8, 298, 1, 4, 1, 0, True, 3, "bf16"),    # rows too long for the whole-sample kernel:
    (2, 24, 16, 700, 2, 4, 3, 1, True, 1, "f32"),    #   channel-first on transposed copies in the workspace
])
def test_bwd_channel_last(B, D, N, T, B2, K, P, act, sp, flags, io):
    """Channel-last backward: bit-identical to channel-first on the transposed tensors
    (and channel-first is checked against the oracle in the same call)."""
    run_case(B=B, D=D, N=N, T=T, B2=B2, K=max(K, 1), P=P, act=act, softplus=sp, flags=flags, io=io, seed=B + T,
             use_conv=K > 0, cl=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_pad_bwd_channel_last(io):
    import torch
    rng = np.random.default_rng(9)
    B, D, T = 3, 72, 13
    g32 = rng.standard_normal((B, D, T + 2)).astype(np.float32)
    g = synth.f32_to_bf16_bits(g32) if io == "bf16" else g32
    cf = sfm.sfm_aux_pad_bwd(to_dev(g))
    cl = sfm.sfm_aux_pad_bwd_ex(to_dev(g).transpose(1, 2).contiguous(), flags=sfm.SFM_LAYOUT_BLD)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(cl.transpose(1, 2).contiguous()), from_dev(cf))


def test_bwd_channel_last_rejects_unaligned_rows():
    import torch
    B, D, N, L = 2, 6, 4, 10  # 6 bf16 channels = 12 bytes per position row
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda")
    with pytest.raises(sfm.SFMError):
        sfm.sfm_selective_scan_bwd(z(B, L, D), z(B, L, D), z(D, N, dt=torch.float32), z(B, L, N), z(B, L, N),
                                   z(B, L, D), conv_w=z(D, 4, dt=torch.float32), flags=sfm.SFM_LAYOUT_BLD)


def test_bwd_long_rows_channel_last_bf16():
    """Channel-last rows of 4002 positions (N = 16): transposed into the workspace,
    the chunked split-row backward, transposed back; bit-identical to channel-first."""
    run_case(B=2, D=128, N=16, T=4000, B2=1, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=37, cl=True)


def test_bwd_long_rows_bf16():
    """Rows of 4002 positions (the long workload's length, N = 16), chunked kernel."""
    run_case(B=2, D=128, N=16, T=4000, B2=1, K=4, P=1, act=0, softplus=True, flags=3, io="bf16", seed=31)
