"""Parity of the streaming lane-split forward kernel (one state per lane, 16
lanes per channel, x / delta / B / C all streamed through LDS in chunks)
against the CPU oracle, through the C ABI.

The planner picks this kernel for long rows with 9 to 16 states (the long
workload); SFM_SCAN_SPLIT=16 forces it on small shapes here, and
SFM_SCAN_SPLIT_CHUNK sets its chunk length, so that every feature is covered:
ragged last chunks, rows shorter than a chunk or than a lane group, folded
rows (the chunks of several samples form one stream), conv widths and
pad_left (left, right and causal halos across chunk edges), SiLU, conv bias,
no conv, no softplus, state counts padded up to 16, partial waves and
workgroups, the fused aux pad and swap (ends in one chunk or two), f32 and bf16
io.  Bars as everywhere: bit-exact for the integer and identity scans and for
fused vs unfused, |g - r| <= rtol (|r| + rms r) against the oracle otherwise.
"""
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from helpers import assert_close, from_dev, to_dev
from test_gpu_split import _int_inputs, env, make, up

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SHAPES = [
    # B, D, N, T, B2, K, P, act, bias, io, chunk
    (2, 64, 16, 298, 1, 4, 1, None, False, "bf16", 128),   # three chunks, the last ragged (44 positions)
    (2, 64, 16, 298, 2, 4, 1, "silu", True, "bf16", 32),   # folded rows: 20 chunks in one stream
    (3, 70, 12, 62, 3, 8, 3, None, True, "f32", 16),       # partial wave and workgroup, widest conv, N -> 16
    (2, 16, 9, 30, 1, 3, 0, None, False, "f32", 16),       # N = 9, right halo (pad_left 0), two chunks
    (2, 8, 16, 1, 1, 4, 1, None, False, "f32", 16),        # L = 3: fewer positions than a lane group
    (2, 64, 16, 14, 1, 2, 1, "silu", False, "bf16", 16),   # L = 16: exactly one block
    (2, 40, 16, 126, 1, 5, 4, None, True, "bf16", 64),     # causal halo, the swapped ends in two chunks
    (2, 4, 16, 254, 2, 4, 1, None, False, "bf16", 256),    # one wave per workgroup, one chunk per sample
    (2, 24, 16, 45, 1, 4, 2, None, False, "f32", 32),      # odd L (f32 words are single elements)
]


def _run(x, delta, Bm, Cm, A, Dk, db, cw, cb, P, act, B2, flags, chunk, y=None):
    import torch
    Tt = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    B, D, T = x.shape
    N, L = Bm.shape[1], T + 2
    K = cw.shape[1]
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=chunk):
        io = "bf16" if x.dtype == np.uint16 else "f32"
        plan = sfm.sfm_scan_plan_string(B // B2, B2, D, N, L, K, io, flags)
        assert f"split=16 chunk={min(chunk, (L + 15) // 16 * 16)}" in plan, plan
        u = xd if flags & 1 else sfm.sfm_aux_pad_swap(xd, mode="pad")
        if y is None:
            y = torch.full((B, D, L), float("nan"), dtype=xd.dtype, device="cuda")
        sfm.sfm_selective_scan_fwd_ex(u, dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db), conv_w=Tt(cw),
                                      conv_b=None if cb is None else Tt(cb), conv_pad_left=P, conv_act=act,
                                      y=y, B2=B2, flags=flags)
        torch.cuda.synchronize()
    return from_dev(y)


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,bias,io,chunk", SHAPES)
@pytest.mark.parametrize("flags", [0, 3])
def test_stream_against_oracle(B, D, N, T, B2, K, P, act, bias, io, chunk, flags):
    say(f"stream B={B} D={D} N={N} T={T} B2={B2} K={K} P={P} act={act} io={io} chunk={chunk} flags={flags}")
    x, delta, Bm, Cm, A, Dk, db, cw, cb = make(B, D, N, T, K, io, seed=B * 3 + D + N + T + K + chunk, bias=bias)
    want = oracle.layer(oracle.aux_pad(up(x), io), up(delta), A, up(Bm), up(Cm), Dk, db, cw, cb, pad_left=P,
                        act=1 if act == "silu" else 0)
    got = _run(x, delta, Bm, Cm, A, Dk, db, cw, cb, P, act, B2, flags, chunk)
    if flags & 2:
        want = oracle.aux_swap(want)
    assert_close(got, want, io, f"stream chunk={chunk}")


@pytest.mark.parametrize("B,D,N,T,B2,K,P,io,chunk", [
    (2, 64, 16, 298, 2, 4, 1, "bf16", 64),   # eight waves per workgroup, folded rows
    (3, 70, 12, 62, 3, 8, 3, "f32", 16),     # three groups, the last one holding 2 of its 8 tiles (1 partial)
    (2, 40, 16, 510, 1, 4, 0, "bf16", 240),  # the long rows' chunk length: interior chunks on the precomputed path
])
@pytest.mark.parametrize("flags", [0, 3])
def test_stream_eight_waves_per_group(B, D, N, T, B2, K, P, io, chunk, flags):
    """Eight waves (32 channels) sharing one B/C stage, as planned for the long rows."""
    say(f"stream wpg=8 B={B} D={D} N={N} T={T} B2={B2} K={K} P={P} io={io} chunk={chunk} flags={flags}")
    x, delta, Bm, Cm, A, Dk, db, cw, cb = make(B, D, N, T, K, io, seed=B + D + N + T + chunk + flags, bias=True)
    want = oracle.layer(oracle.aux_pad(up(x), io), up(delta), A, up(Bm), up(Cm), Dk, db, cw, cb, pad_left=P)
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=chunk, SFM_SCAN_SPLIT_WPG=8):
        assert "wpg=8" in sfm.sfm_scan_plan_string(B // B2, B2, D, N, T + 2, K, io, flags)
        got = _run(x, delta, Bm, Cm, A, Dk, db, cw, cb, P, None, B2, flags, chunk)
    if flags & 2:
        want = oracle.aux_swap(want)
    assert_close(got, want, io, f"stream wpg=8 chunk={chunk}")


@pytest.mark.parametrize("softplus", [True, False])
def test_stream_no_conv(softplus):
    import torch
    B, D, N, T, io = 3, 20, 16, 100, "f32"
    L = T + 2
    x, delta, Bm, Cm, A, Dk, db, _, _ = make(B, D, N, T, 1, io, seed=40 + softplus)
    if not softplus:
        delta = np.abs(delta)
        db = np.zeros_like(db)
    u = oracle.aux_pad(up(x), io).astype(np.float32)
    Tt = lambda a: torch.from_numpy(a).cuda()
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=32):
        assert "split=16 chunk=32" in sfm.sfm_scan_plan_string(B, 1, D, N, L, 0, io, 0)
        y = sfm.sfm_selective_scan_fwd(to_dev(u), to_dev(delta), Tt(A), to_dev(Bm), to_dev(Cm), Tt(Dk), Tt(db),
                                       delta_softplus=softplus, B2=1)
        torch.cuda.synchronize()
    want = oracle.selective_scan(u.astype(np.float64), up(delta), A, up(Bm), up(Cm), Dk, db, softplus=softplus)
    assert_close(from_dev(y), want, io, "stream no conv")


@pytest.mark.parametrize("N", [9, 16])
@pytest.mark.parametrize("B2", [1, 2])
def test_stream_integer_scan_counts_positions(N, B2):
    """A = 0, Delta = 1, B = C = 1, D = 0, u = 1  =>  y[b,d,t] = N (t + 1) exactly, across chunks and samples."""
    import torch
    B, D, L = 4, 36, 300
    a = _int_inputs(B, D, L, N, 0.0)
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=32):
        assert "split=16 chunk=32" in sfm.sfm_scan_plan_string(B // B2, B2, D, N, L, 0, "f32", 0)
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=B2)
        torch.cuda.synchronize()
    want = np.broadcast_to(N * np.arange(1, L + 1, dtype=np.float64), (B, D, L))
    assert np.array_equal(from_dev(y), want)


def test_stream_identity_scan():
    """A = -inf (Abar = 0), N = 16, B = C = 1, Delta = 1: y = N * u exactly for integer u."""
    import torch
    B, D, L, N = 2, 12, 140, 16
    u = torch.arange(B * D * L, dtype=torch.float32, device="cuda").reshape(B, D, L) + 1
    a = _int_inputs(B, D, L, N, float("-inf"), u=u)
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=64):
        assert "split=16" in sfm.sfm_scan_plan_string(B, 1, D, N, L, 0, "f32", 0)
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=1)
        torch.cuda.synchronize()
    assert np.array_equal(from_dev(y), 16.0 * from_dev(u))


def test_stream_reset_isolates_poisoned_sample():
    B, D, N, T, K, io = 4, 16, 16, 94, 4, "f32"
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=77)

    def run(xx, dl):
        return _run(xx, dl, Bm, Cm, A, Dk, db, cw, None, 1, None, 4, 3, 32)

    clean = run(x, delta)
    for poison in (np.nan, np.inf, 1e30):
        xx, dl = x.copy(), delta.copy()
        xx[1] = poison
        dl[1] = poison
        got = run(xx, dl)
        assert np.array_equal(got[[0, 2, 3]], clean[[0, 2, 3]]), f"poison {poison} leaked"


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_stream_fused_matches_unfused_chain(flags):
    """Fused pad/swap on the streaming kernel is bit-identical to pad -> scan -> swap
    (bf16 rows: the float64 piece sums of the row mean are exact)."""
    import torch
    B, D, N, T, B2, K, P, io = 3, 36, 16, 254, 3, 4, 1, "bf16"
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=flags + 60)
    Tt = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    with env(SFM_SCAN_SPLIT=16, SFM_SCAN_SPLIT_CHUNK=64):
        xp = sfm.sfm_aux_pad_swap(xd, mode="pad")
        ref = sfm.sfm_selective_scan_fwd(xp, dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db), conv_w=Tt(cw), conv_pad_left=P,
                                         B2=B2)
        if flags & 2:
            sfm.sfm_aux_pad_swap(ref, out=ref, mode="swap")
        got = sfm.sfm_selective_scan_fwd_ex(xd if flags & 1 else xp, dd, Tt(A), Bd, Cd, Tt(Dk), Tt(db),
                                            conv_w=Tt(cw), conv_pad_left=P, B2=B2, flags=flags)
        torch.cuda.synchronize()
    assert np.array_equal(from_dev(got), from_dev(ref))


def test_stream_deterministic_and_every_element_written():
    B, D, N, T, K, io = 4, 52, 16, 510, 4, "bf16"
    x, delta, Bm, Cm, A, Dk, db, cw, _ = make(B, D, N, T, K, io, seed=8)
    outs = [_run(x, delta, Bm, Cm, A, Dk, db, cw, None, 1, None, 2, 3, 128) for _ in range(2)]
    assert not np.isnan(outs[0]).any()
    assert np.array_equal(outs[0], outs[1])


def test_planner_streams_long_rows():
    """The long workload (16 samples x 320 channels x 4002 positions, 16 states):
    80 one-lane waves for 1024 SIMDs, rows too long to stage whole -> the
    streaming kernel, 1280 waves, with the longest chunk that keeps every
    workgroup resident at once."""
    with env(SFM_SCAN_SPLIT=-1, SFM_SCAN_SPLIT_CHUNK=-1):
        plan = sfm.sfm_scan_plan_string(16, 1, 320, 16, 4002, 4, "bf16", 3)
        assert "split=16 chunk=240 ns=16 wpg=8" in plan and "grid=160 block=512" in plan, plan
