"""Parity of the lane-split forward kernel (N states of a channel spread over
2 or 4 lanes) against the CPU oracle, through the C ABI.

The planner picks this kernel for whole-row shapes that fill the GPU; here
SFM_SCAN_SPLIT forces it (and its lane-group size) on small shapes too, so every
feature of the launch is covered: conv widths and pad_left, SiLU, conv bias,
no conv, no softplus, state counts padded up to 4/8/16, row lengths that do
not divide into the lane groups, partial channel tiles, folded rows (B2 > 1),
the fused aux pad and swap, f32 and bf16 io.  Bars as everywhere: bit-exact
for the integer and identity scans, |g - r| <= rtol (|r| + rms r) otherwise.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        for k, v in self.kv.items():
            os.environ[k] = str(v)

    def __exit__(self, *a):
        for k, v in self.old.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v


def up(a):
    return synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def make(B, D, N, T, K, io, seed, bias=False):
    r = np.random.default_rng(seed)
    L = T + 2
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    cast = synth.f32_to_bf16_bits if io == "bf16" else (lambda a: a)
    x, delta, Bm, Cm = map(cast, (f(B, D, T), f(B, D, L), f(B, N, L), f(B, N, L)))
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk, db = f(D), r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, max(K, 1))).astype(np.float32)
    cb = f(D) if bias else None
    return x, delta, Bm, Cm, A, Dk, db, cw, cb


SHAPES = [
    # B, D, N, T, B2, K, P, act, bias, io, G
    (4, 64, 8, 49, 1, 4, 1, None, False, "bf16", 2),    # stage-4 shape, small batch
    (4, 64, 8, 49, 2, 4, 1, None, False, "bf16", 4),
    (3, 96, 5, 30, 3, 4, 1, None, True, "bf16", 2),     # N padded to 8, partial workgroup, B2 = B
    (2, 128, 16, 20, 1, 8, 3, "silu", True, "f32", 2),  # 16 states, widest conv, causal-ish pad
    (2, 128, 16, 21, 2, 3, 0, None, False, "f32", 4),   # odd L with G = 4 (ragged last block)
    (2, 64, 3, 6, 1, 1, 0, None, False, "f32", 2),      # K = 1, N padded to 4, L = 8
    (2, 64, 12, 1, 2, 2, 1, "silu", False, "f32", 4),   # T = 1 (L = 3), fewer positions than G
    (4, 64, 8, 196, 2, 4, 1, None, False, "bf16", 4),   # stage-3 row length
    (2, 96, 8, 62, 1, 5, 4, None, True, "bf16", 4),     # right-only halo (P = K-1)
    (3, 72, 8, 49, 1, 4, 1, None, False, "bf16", 2),    # partial wave: 8 of 32 channels
    (3, 72, 8, 49, 3, 4, 1, "silu", True, "bf16", 4),   # partial wave: 8 of 16 channels
    (4, 16, 4, 8, 2, 4, 1, None, False, "f32", 2),      # the tiny workload: one wave, 16 of 32 channels
]


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,bias,io,G", SHAPES)
@pytest.mark.parametrize("flags", [0, 3])
def test_split_against_oracle(B, D, N, T, B2, K, P, act, bias, io, G, flags):
    import torch
    say(f"split B={B} D={D} N={N} T={T} B2={B2} K={K} P={P} act={act} io={io} G={G} flags={flags}")
    L = T + 2
    x, delta, Bm, Cm, A, Dk, db, cw, cb = make(B, D, N, T, K, io, seed=B * 7 + D + N + T + K, bias=bias)
    Tt = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    xp64 = oracle.aux_pad(up(x), io)
    want = oracle.layer(xp64, up(delta), A, up(Bm), up(Cm), Dk, db, cw, cb, pad_left=P,
                        act=1 if act == "silu" else 0)
    with env(SFM_SCAN_SPLIT=G):
        plan = sfm.sfm_scan_plan_string(B // B2, B2, D, N, L, K, io, flags)
        assert f"split={G}" in plan, plan
        if flags & 1:
            u = xd
        else:
            u = sfm.sfm_aux_pad_swap(xd, mode="pad")
        y = sfm.sfm_selective_scan_fwd_ex(u, dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db), conv_w=Tt(cw),
                                          conv_b=None if cb is None else Tt(cb), conv_pad_left=P, conv_act=act,
                                          B2=B2, flags=flags)
        torch.cuda.synchronize()
    got = from_dev(y)
    if flags & 2:
        want = oracle.aux_swap(want)
    assert_close(got, want, io, f"split G={G}")


@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("T,io", [(49, "bf16"), (196, "bf16"), (21, "f32"), (3, "bf16"), (1, "f32")])
def test_split_fused_pad_matches_the_pad_kernel(G, T, io):
    """The fused aux pad of the whole-row kernel takes each row's mean as G
    piece sums (lane g of a channel sums piece g in float64, in index order)
    added in piece order: on rows whose float64 partial sums are exact it is
    the pad kernel's index-order mean, so the fused step is bit-identical to
    pad + scan + swap as three launches.  Pieces of unequal length (T not a
    multiple of G) and rows shorter than the lane group (empty pieces)."""
    import torch
    B, D, N, K = 3, 96, 8, 4
    L = T + 2
    say(f"split fused pad G={G} T={T} io={io}")
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=G * 100 + T)
    Tt = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    with env(SFM_SCAN_SPLIT=G, SFM_SCAN_SPLIT_CHUNK=0):  # whole rows
        plan = sfm.sfm_scan_plan_string(B, 1, D, N, L, K, io, 3)
        assert f"split={G} chunk=0" in plan, plan
        args = (dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db))
        fused = sfm.sfm_selective_scan_fwd_ex(xd, *args, conv_w=Tt(cw), conv_pad_left=1, flags=3)
        xp = sfm.sfm_aux_pad_swap(xd, mode="pad")
        y = sfm.sfm_selective_scan_fwd_ex(xp, *args, conv_w=Tt(cw), conv_pad_left=1, flags=0)
        sfm.sfm_aux_pad_swap(y, out=y, mode="swap")
        torch.cuda.synchronize()
    assert np.array_equal(from_dev(fused), from_dev(y))


@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("softplus", [True, False])
def test_split_no_conv(G, softplus):
    import torch
    B, D, N, T, io = 3, 64, 8, 38, "f32"
    L = T + 2
    x, delta, Bm, Cm, A, Dk, db, _, _ = make(B, D, N, T, 1, io, seed=G + 10 * softplus)
    if not softplus:
        delta = np.abs(delta)
        db = np.zeros_like(db)
    u = oracle.aux_pad(up(x), io).astype(np.float32)
    Tt = lambda a: torch.from_numpy(a).cuda()
    with env(SFM_SCAN_SPLIT=G):
        assert f"split={G}" in sfm.sfm_scan_plan_string(B, 1, D, N, L, 0, io, 0)
        y = sfm.sfm_selective_scan_fwd(to_dev(u), to_dev(delta), Tt(A), to_dev(Bm), to_dev(Cm), Tt(Dk), Tt(db),
                                       delta_softplus=softplus, B2=1)
        torch.cuda.synchronize()
    want = oracle.selective_scan(u.astype(np.float64), up(delta), A, up(Bm), up(Cm), Dk, db, softplus=softplus)
    assert_close(from_dev(y), want, io, f"split no conv G={G}")


def _int_inputs(B, D, L, N, a_val, u=None):
    import torch
    dev = "cuda"
    u = torch.ones((B, D, L), device=dev) if u is None else u
    return dict(u=u, delta=torch.ones((B, D, L), device=dev), A=torch.full((D, N), a_val, device=dev),
                Bm=torch.ones((B, N, L), device=dev), Cm=torch.ones((B, N, L), device=dev),
                Dskip=torch.zeros(D, device=dev), delta_bias=torch.zeros(D, device=dev))


@pytest.mark.parametrize("G,N", [(2, 1), (4, 5)])
@pytest.mark.parametrize("B2", [1, 4])
def test_split_integer_scan_counts_positions(G, N, B2):
    """A = 0, Delta = 1, B = C = 1, D = 0, u = 1  =>  y[b,d,t] = N (t + 1) exactly."""
    import torch
    B, D, L = 8, 128, 36
    a = _int_inputs(B, D, L, N, 0.0)
    with env(SFM_SCAN_SPLIT=G):
        assert f"split={G}" in sfm.sfm_scan_plan_string(B // B2, B2, D, N, L, 0, "f32", 0)
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=B2)
        torch.cuda.synchronize()
    want = np.broadcast_to(N * np.arange(1, L + 1, dtype=np.float64), (B, D, L))
    assert np.array_equal(from_dev(y), want)


@pytest.mark.parametrize("G", [2, 4])
def test_split_identity_scan(G):
    """A = -inf (Abar = 0), N = 8, B = C = 1, Delta = 1: y = N * u exactly for integer u."""
    import torch
    B, D, L, N = 4, 64, 24, 8
    u = torch.arange(B * D * L, dtype=torch.float32, device="cuda").reshape(B, D, L) + 1
    a = _int_inputs(B, D, L, N, float("-inf"), u=u)
    with env(SFM_SCAN_SPLIT=G):
        assert f"split={G}" in sfm.sfm_scan_plan_string(B, 1, D, N, L, 0, "f32", 0)
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=1)
        torch.cuda.synchronize()
    assert np.array_equal(from_dev(y), 8.0 * from_dev(u))


@pytest.mark.parametrize("G", [2, 4])
def test_split_reset_isolates_poisoned_sample(G):
    import torch
    B, D, N, T, K, io = 4, 64, 8, 30, 4, "f32"
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=99)
    Tt = lambda a: torch.from_numpy(a).cuda()

    def run(xx, dl):
        with env(SFM_SCAN_SPLIT=G):
            y = sfm.sfm_selective_scan_fwd_ex(to_dev(xx), to_dev(dl), Tt(A), to_dev(Bm), to_dev(Cm), Tt(Dk), Tt(db),
                                              conv_w=Tt(cw), conv_pad_left=1, B2=4, flags=3)
            torch.cuda.synchronize()
        return from_dev(y)

    clean = run(x, delta)
    for poison in (np.nan, np.inf, 1e30):
        xx, dl = x.copy(), delta.copy()
        xx[1] = poison
        dl[1] = poison
        got = run(xx, dl)
        assert np.array_equal(got[[0, 2, 3]], clean[[0, 2, 3]]), f"poison {poison} leaked"


def test_split_deterministic_and_every_element_written():
    import torch
    B, D, N, T, K, io = 8, 192, 8, 49, 4, "bf16"
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=5)
    Tt = lambda a: torch.from_numpy(a).cuda()
    outs = []
    for _ in range(2):
        y = torch.full((B, D, T + 2), float("nan"), dtype=torch.bfloat16, device="cuda")
        with env(SFM_SCAN_SPLIT=2):
            sfm.sfm_selective_scan_fwd_ex(to_dev(x), to_dev(delta), Tt(A), to_dev(Bm), to_dev(Cm), Tt(Dk), Tt(db),
                                          conv_w=Tt(cw), conv_pad_left=1, y=y, B2=2, flags=3)
            torch.cuda.synchronize()
        outs.append(from_dev(y))
    assert not np.isnan(outs[0]).any()
    assert np.array_equal(outs[0], outs[1])


def test_planner_picks_the_kernel_by_waves_per_simd():
    """One wave per (sample, 64-channel tile): 1280 at stage-3 (1.25 per SIMD:
    four lanes per channel, at any fold), 2560 at stage-4 (2.5 per SIMD: two
    lanes per channel unfolded, the one-lane kernel folded), 4096 at the base
    model's stage-3 (4 per SIMD: two lanes per channel unfolded)."""
    with env(SFM_SCAN_SPLIT=-1):
        assert "split=4" in sfm.sfm_scan_plan_string(256, 1, 320, 8, 198, 4, "bf16", 3)
        assert "split=4" in sfm.sfm_scan_plan_string(64, 4, 320, 8, 198, 4, "bf16", 3)
        assert "split=2" in sfm.sfm_scan_plan_string(256, 1, 640, 8, 51, 4, "bf16", 3)
        assert "mode=" in sfm.sfm_scan_plan_string(64, 4, 640, 8, 51, 4, "bf16", 3)
        assert "split=2" in sfm.sfm_scan_plan_string(512, 1, 512, 16, 198, 4, "bf16", 3)
        assert "mode=" in sfm.sfm_scan_plan_string(128, 4, 512, 16, 198, 4, "bf16", 3)


CHUNK_SHAPES = [
    # B, D, N, T, B2, K, P, act, bias, io, G, chunk
    (4, 64, 8, 196, 1, 4, 1, None, False, "bf16", 4, 24),    # stage-3 rows, ragged last chunk (6 positions)
    (4, 64, 8, 196, 2, 4, 1, "silu", True, "bf16", 2, 32),   # two lanes per channel, folded rows
    (3, 72, 16, 62, 3, 8, 3, None, True, "f32", 4, 16),      # partial wave, widest conv, 16 states
    (2, 64, 5, 30, 2, 3, 0, None, False, "f32", 4, 16),      # two chunks, N padded to 8
    (2, 64, 8, 1, 1, 4, 1, None, False, "f32", 4, 16),       # L = 3: one chunk shorter than the chunk size
    (2, 128, 8, 46, 1, 4, 2, None, False, "bf16", 4, 48),    # one chunk holding both swapped ends
    (2, 64, 8, 25, 1, 4, 1, None, False, "f32", 4, 16),      # odd L (f32 words are single elements)
]


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,bias,io,G,chunk", CHUNK_SHAPES)
@pytest.mark.parametrize("flags", [0, 3])
def test_split_chunked_against_oracle(B, D, N, T, B2, K, P, act, bias, io, G, chunk, flags):
    """The chunked staging (x whole rows; delta/y and raw B/C in chunks)."""
    import torch
    say(f"split chunked B={B} D={D} N={N} T={T} B2={B2} K={K} io={io} G={G} chunk={chunk} flags={flags}")
    L = T + 2
    x, delta, Bm, Cm, A, Dk, db, cw, cb = make(B, D, N, T, K, io, seed=B * 5 + D + N + T + chunk, bias=bias)
    Tt = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    xp64 = oracle.aux_pad(up(x), io)
    want = oracle.layer(xp64, up(delta), A, up(Bm), up(Cm), Dk, db, cw, cb, pad_left=P,
                        act=1 if act == "silu" else 0)
    with env(SFM_SCAN_SPLIT=G, SFM_SCAN_SPLIT_CHUNK=chunk):
        plan = sfm.sfm_scan_plan_string(B // B2, B2, D, N, L, K, io, flags)
        assert f"split={G} chunk={min(chunk, (L + 3) // 4 * 4)}" in plan, plan
        u = xd if flags & 1 else sfm.sfm_aux_pad_swap(xd, mode="pad")
        y = torch.full((B, D, L), float("nan"), dtype=xd.dtype, device="cuda")
        sfm.sfm_selective_scan_fwd_ex(u, dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db), conv_w=Tt(cw),
                                      conv_b=None if cb is None else Tt(cb), conv_pad_left=P, conv_act=act,
                                      y=y, B2=B2, flags=flags)
        torch.cuda.synchronize()
    got = from_dev(y)
    if flags & 2:
        want = oracle.aux_swap(want)
    assert_close(got, want, io, f"split chunked G={G} chunk={chunk}")


@pytest.mark.parametrize("G,N", [(2, 1), (4, 5)])
def test_split_chunked_integer_scan(G, N):
    """A = 0, Delta = 1, B = C = 1, D = 0, u = 1  =>  y = N (t + 1) exactly, chunk by chunk."""
    import torch
    B, D, L = 4, 64, 70
    a = _int_inputs(B, D, L, N, 0.0)
    with env(SFM_SCAN_SPLIT=G, SFM_SCAN_SPLIT_CHUNK=16):
        assert f"split={G} chunk=16" in sfm.sfm_scan_plan_string(B, 1, D, N, L, 0, "f32", 0)
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=2)
        torch.cuda.synchronize()
    want = np.broadcast_to(N * np.arange(1, L + 1, dtype=np.float64), (B, D, L))
    assert np.array_equal(from_dev(y), want)


def test_planner_keeps_whole_rows_where_they_fit():
    """Stage-3 rows fit whole (two waves per SIMD resident); the chunked staging is
    used only when asked for (or when whole rows would not keep two per SIMD)."""
    with env(SFM_SCAN_SPLIT=-1):
        assert "split=4 chunk=0" in sfm.sfm_scan_plan_string(256, 1, 320, 8, 198, 4, "bf16", 3)
