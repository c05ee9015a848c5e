"""Parity of sfm_selective_scan_fwd_ws (rows split along L across segment waves,
carries composed in a second pass) through the C ABI against the float64 oracle,
with the forward's tolerance: |g - r| <= rtol (|r| + rms r), rtol 1e-5 with f32
io and 2e-2 with bf16 io.  Segment counts are forced with SFM_BWD_SEGMENTS at
small sizes (every boundary case: the pad's mean, the swap, conv windows reaching
across segments); the long workload's rows take the default split."""
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import assert_close, from_dev, host_threads, to_dev

pytestmark = pytest.mark.gpu
NT = host_threads()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(B, D, N, T, K, P, act, flags, io, seed, conv=True, samples=None, B2=1):
    import torch
    w = synth.Workload("fws", B=B, D=D, N=N, T=T, io=io, B2_list=(1,), K=max(K, 1))
    li = synth.make_layer(w, seed=seed)
    L = T + 2
    pad = bool(flags & sfm.SFM_FUSE_PAD)
    f64 = (lambda a: synth.bf16_bits_to_f64(a)) if io == "bf16" else (lambda a: a.astype(np.float64))
    x = li.x
    if not pad:
        rng = np.random.default_rng(seed + 5)
        xr = rng.standard_normal((B, D, L)).astype(np.float32)
        x = synth.f32_to_bf16_bits(xr) if io == "bf16" else xr
    cw = li.conv_w[:, :K] if conv else None
    need = sfm.sfm_selective_scan_fwd_ws_size(B // B2, B2, D, N, L, K if conv else 0, io, flags)
    say(f"fwd_ws B={B} D={D} N={N} T={T} K={K} P={P} act={act} flags={flags} io={io} workspace={need}")
    assert need > 0, "the plan must split the rows"
    got = sfm.sfm_selective_scan_fwd_ws(to_dev(x), to_dev(li.delta), torch.from_numpy(li.A).cuda(),
                                        to_dev(li.Bm), to_dev(li.Cm), torch.from_numpy(li.Dskip).cuda(),
                                        torch.from_numpy(li.delta_bias).cuda(),
                                        conv_w=torch.from_numpy(np.ascontiguousarray(cw)).cuda() if conv else None,
                                        conv_pad_left=P, conv_act="silu" if act else None, B2=B2, flags=flags)
    torch.cuda.synchronize()
    sel = slice(None) if samples is None else samples
    xo = f64(x)
    if pad:
        xo = oracle.aux_pad(xo, io)
    xo = xo[sel]
    args = (f64(li.delta)[sel], li.A.astype(np.float64), f64(li.Bm)[sel], f64(li.Cm)[sel],
            li.Dskip.astype(np.float64), li.delta_bias.astype(np.float64))
    if conv:
        want = oracle.layer(xo, *args, cw.astype(np.float64), pad_left=P, act=act, nthreads=NT)
    else:
        want = oracle.selective_scan(xo, *args, nthreads=NT)
    if flags & sfm.SFM_FUSE_SWAP:
        want = oracle.aux_swap(want)
    assert_close(from_dev(got)[sel], want, io, f"fwd_ws {B}x{D}x{L}")
    return got


@pytest.mark.parametrize("B,D,N,T,K,P,act,flags,segs,conv", [
    (2, 70, 5, 60, 4, 1, 1, 3, 3, True),     # pad and swap, partial tile, N padded to 8, SiLU
    (2, 24, 16, 45, 4, 3, 0, 0, 4, True),    # causal conv, N = 16
    (1, 16, 4, 40, 8, 2, 0, 3, 5, True),     # widest window, lag 5
    (2, 16, 8, 30, 4, 0, 0, 1, 3, True),     # pad only, anti-causal window
    (2, 16, 4, 30, 1, 0, 0, 2, 4, False),    # no conv, swap only
])
def test_fwd_ws_forced_segments_f32(B, D, N, T, K, P, act, flags, segs, conv, monkeypatch):
    monkeypatch.setenv("SFM_BWD_SEGMENTS", str(segs))
    run(B, D, N, T, K, P, act, flags, "f32", seed=B * 13 + T, conv=conv)


def test_fwd_ws_folded_rows_f32(monkeypatch):
    """Folded rows (B2 = 2): the split path runs every sample as its own row, as the
    reset makes them independent."""
    monkeypatch.setenv("SFM_BWD_SEGMENTS", "3")
    run(4, 40, 8, 70, 4, 1, 0, 3, "f32", seed=23, B2=2)


def test_fwd_ws_long_rows_bf16():
    """Long rows (L = 4002) of 8 states, which only the split-row scheme spreads
    over the GPU, with the default split, two samples."""
    run(2, 128, 8, 4000, 4, 1, 0, 3, "bf16", seed=17)


def test_fwd_ws_streamed_rows_take_the_regular_forward():
    """Long rows of 16 states (the long workload's shape, two samples): the regular
    forward streams them faster than the split-row scheme, so the workspace entry
    point needs no workspace and gives the regular forward's bits."""
    import torch
    B, D, N, T = 2, 128, 16, 4000
    assert sfm.sfm_selective_scan_fwd_ws_size(B, 1, D, N, T + 2, 4, "bf16", 3) == 0
    assert "split=16" in sfm.sfm_scan_plan_string(B, 1, D, N, T + 2, 4, "bf16", 3)
    w = synth.Workload("fws", B=B, D=D, N=N, T=T, io="bf16", B2_list=(1,), K=4)
    li = synth.make_layer(w, seed=19)
    args = (to_dev(li.x), to_dev(li.delta), torch.from_numpy(li.A).cuda(), to_dev(li.Bm), to_dev(li.Cm),
            torch.from_numpy(li.Dskip).cuda(), torch.from_numpy(li.delta_bias).cuda())
    kw = dict(conv_w=torch.from_numpy(li.conv_w).cuda(), conv_pad_left=1, flags=3)
    a = sfm.sfm_selective_scan_fwd_ws(*args, **kw)
    b = sfm.sfm_selective_scan_fwd_ex(*args, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(a), from_dev(b))


def test_fwd_ws_falls_back_without_split():
    """Shapes the plan does not split report a zero workspace and run the regular forward."""
    import torch
    assert sfm.sfm_selective_scan_fwd_ws_size(256, 1, 640, 8, 51, 4, "bf16", 3) == 0
    w = synth.WORKLOADS["tiny"]
    li = synth.make_layer(w, seed=3)
    args = (to_dev(li.x), to_dev(li.delta), torch.from_numpy(li.A).cuda(), to_dev(li.Bm), to_dev(li.Cm),
            torch.from_numpy(li.Dskip).cuda(), torch.from_numpy(li.delta_bias).cuda())
    kw = dict(conv_w=torch.from_numpy(li.conv_w).cuda(), conv_pad_left=1, flags=3)
    a = sfm.sfm_selective_scan_fwd_ws(*args, **kw)
    b = sfm.sfm_selective_scan_fwd_ex(*args, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(a), from_dev(b))
